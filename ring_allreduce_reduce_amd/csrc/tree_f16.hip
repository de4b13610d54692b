// Tree AllReduce kernels for one element type (one translation unit per
// type so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP, bool CAP>
static const void* tree_by_proto_f16(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&tree_kernel<F16, OP, kLL, true, CAP>
                                 : (const void*)&tree_kernel<F16, OP, kLL, false, CAP>;
  if (proto == kLL128) return (const void*)&tree_kernel<F16, OP, kLL128, false, CAP>;
  return small ? (const void*)&tree_kernel<F16, OP, kSimple, true, CAP>
               : (const void*)&tree_kernel<F16, OP, kSimple, false, CAP>;
}

template <bool CAP>
static const void* tree_by_op_f16(int op, int proto, bool small) {
  switch (op) {
    case 0: return tree_by_proto_f16<0, CAP>(proto, small);
    case 1: return tree_by_proto_f16<1, CAP>(proto, small);
    case 2: return tree_by_proto_f16<2, CAP>(proto, small);
    case 3: return tree_by_proto_f16<3, CAP>(proto, small);
    default: return tree_by_proto_f16<4, CAP>(proto, small);
  }
}

const void* kernel_tree_for_f16(int op, int proto, bool small, bool cap) {
  return cap ? tree_by_op_f16<true>(op, proto, small) : tree_by_op_f16<false>(op, proto, small);
}

}  // namespace ringar
