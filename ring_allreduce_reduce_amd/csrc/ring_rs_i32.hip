// Ring ReduceScatter kernels for one element type (one translation unit per type
// so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP>
static const void* by_proto_kernel_rs_i32(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&ring_kernel_lines<I32, OP, kLL, true, kReduceScatter>
                                 : (const void*)&ring_kernel_lines<I32, OP, kLL, false, kReduceScatter>;
  if (proto == kLL128) return (const void*)&ring_kernel_lines<I32, OP, kLL128, false, kReduceScatter>;
  return small ? (const void*)&ring_kernel<I32, OP, kSimple, true, kReduceScatter>
               : (const void*)&ring_kernel<I32, OP, kSimple, false, kReduceScatter>;
}

const void* kernel_rs_for_i32(int op, int proto, bool small) {
  switch (op) {
    case 0: return by_proto_kernel_rs_i32<0>(proto, small);
    case 1: return by_proto_kernel_rs_i32<1>(proto, small);
    case 2: return by_proto_kernel_rs_i32<2>(proto, small);
    case 3: return by_proto_kernel_rs_i32<3>(proto, small);
    default: return by_proto_kernel_rs_i32<4>(proto, small);
  }
}

}  // namespace ringar
