// Ring ReduceScatter kernels for one element type (one translation unit per type
// so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP, bool CAP>
static const void* by_proto_kernel_rs_f64(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&ring_kernel_lines<F64, OP, kLL, true, kReduceScatter, CAP>
                                 : (const void*)&ring_kernel_lines<F64, OP, kLL, false, kReduceScatter, CAP>;
  if (proto == kLL128) return (const void*)&ring_kernel_lines<F64, OP, kLL128, false, kReduceScatter, CAP>;
  return small ? (const void*)&ring_kernel<F64, OP, kSimple, true, kReduceScatter, CAP>
               : (const void*)&ring_kernel<F64, OP, kSimple, false, kReduceScatter, CAP>;
}

template <bool CAP>
static const void* by_op_kernel_rs_f64(int op, int proto, bool small) {
  switch (op) {
    case 0: return by_proto_kernel_rs_f64<0, CAP>(proto, small);
    case 1: return by_proto_kernel_rs_f64<1, CAP>(proto, small);
    case 2: return by_proto_kernel_rs_f64<2, CAP>(proto, small);
    case 3: return by_proto_kernel_rs_f64<3, CAP>(proto, small);
    default: return by_proto_kernel_rs_f64<4, CAP>(proto, small);
  }
}

const void* kernel_rs_for_f64(int op, int proto, bool small, bool cap) {
  return cap ? by_op_kernel_rs_f64<true>(op, proto, small) : by_op_kernel_rs_f64<false>(op, proto, small);
}

}  // namespace ringar
