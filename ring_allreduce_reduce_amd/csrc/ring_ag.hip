// Ring AllGather kernels: a byte copy, so one instance per protocol (the
// host passes sizes in bytes).
#include "ring_kernel_impl.h"

namespace ringar {

const void* kernel_ag_for(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&ring_kernel_lines<I8, 0, kLL, true, kAllGather>
                                 : (const void*)&ring_kernel_lines<I8, 0, kLL, false, kAllGather>;
  if (proto == kLL128) return (const void*)&ring_kernel_lines<I8, 0, kLL128, false, kAllGather>;
  return small ? (const void*)&ring_kernel<I8, 0, kSimple, true, kAllGather>
               : (const void*)&ring_kernel<I8, 0, kSimple, false, kAllGather>;
}

}  // namespace ringar
