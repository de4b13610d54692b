// Ring ReduceScatter kernels for one element type, eager form (one
// translation unit per type so the instances compile in parallel).
#include "ring_instances.h"

namespace ringar {

const void* kernel_rs_for_bf16(int op, int proto, bool small) {
  return ring_instance_by_op<BF16, kReduceScatter, false>(op, proto, small);
}

}  // namespace ringar
