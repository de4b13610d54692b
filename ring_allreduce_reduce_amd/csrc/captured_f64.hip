// The captured form (stream capture) of every collective for one element
// type: kernel instances that count steps from zero and leave what they
// consumed at zero, kept out of the eager kernels' translation units.
#include "ring_instances.h"

namespace ringar {

const void* kernel_captured_for_f64(int coll, int op, int proto, bool small) {
  if (coll == kTreeAllReduce) return tree_instance_by_op<F64, true>(op, proto, small);
  if (coll == kReduceScatter) return ring_instance_by_op<F64, kReduceScatter, true>(op, proto, small);
  return ring_instance_by_op<F64, kAllReduce, true>(op, proto, small);
}

}  // namespace ringar
