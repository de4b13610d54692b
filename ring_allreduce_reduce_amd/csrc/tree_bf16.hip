// Tree AllReduce kernels for one element type, eager form (one translation
// unit per type so the instances compile in parallel).
#include "ring_instances.h"

namespace ringar {

const void* kernel_tree_for_bf16(int op, int proto, bool small) {
  return tree_instance_by_op<BF16, false>(op, proto, small);
}

}  // namespace ringar
