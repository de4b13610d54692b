// Tree AllReduce kernels for one element type (one translation unit per
// type so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP>
static const void* tree_by_proto_bf16(int proto, bool small) {
  if (proto == kLL) return small ? (const void*)&tree_kernel<BF16, OP, kLL, true>
                                 : (const void*)&tree_kernel<BF16, OP, kLL, false>;
  if (proto == kLL128) return (const void*)&tree_kernel<BF16, OP, kLL128, false>;
  return small ? (const void*)&tree_kernel<BF16, OP, kSimple, true>
               : (const void*)&tree_kernel<BF16, OP, kSimple, false>;
}

const void* kernel_tree_for_bf16(int op, int proto, bool small) {
  switch (op) {
    case 0: return tree_by_proto_bf16<0>(proto, small);
    case 1: return tree_by_proto_bf16<1>(proto, small);
    case 2: return tree_by_proto_bf16<2>(proto, small);
    case 3: return tree_by_proto_bf16<3>(proto, small);
    default: return tree_by_proto_bf16<4>(proto, small);
  }
}

}  // namespace ringar
