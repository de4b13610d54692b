// Ring AllReduce kernels for one element type, eager form (one translation
// unit per type so the instances compile in parallel).
#include "ring_instances.h"

namespace ringar {

const void* kernel_for_i32(int op, int proto, bool small) {
  return ring_instance_by_op<I32, kAllReduce, false>(op, proto, small);
}

}  // namespace ringar
