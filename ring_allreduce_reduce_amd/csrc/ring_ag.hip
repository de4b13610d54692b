// Ring AllGather kernels: a byte copy, so one instance per protocol (the
// host passes sizes in bytes).
#include "ring_kernel_impl.h"

namespace ringar {

template <bool CAP>
static const void* ag_by_proto(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&ring_kernel_lines<I8, 0, kLL, true, kAllGather, CAP>
                                 : (const void*)&ring_kernel_lines<I8, 0, kLL, false, kAllGather, CAP>;
  if (proto == kLL128) return (const void*)&ring_kernel_lines<I8, 0, kLL128, false, kAllGather, CAP>;
  return small ? (const void*)&ring_kernel<I8, 0, kSimple, true, kAllGather, CAP>
               : (const void*)&ring_kernel<I8, 0, kSimple, false, kAllGather, CAP>;
}

const void* kernel_ag_for(int proto, bool small, bool cap) {
  return cap ? ag_by_proto<true>(proto, small) : ag_by_proto<false>(proto, small);
}

}  // namespace ringar
