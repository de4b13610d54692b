// The captured form (stream capture) of every collective for one element
// type: kernel instances that count steps from zero and leave what they
// consumed at zero, kept out of the eager kernels' translation units.
#include "ring_instances.h"

namespace ringar {

const void* kernel_captured_for_i8(int coll, int op, int proto, bool small) {
  // AllGather is a byte copy: its kernels are the int8 ones
  if (coll == kAllGather) return ring_instance<I8, kAllGather, 0, true>(proto, small);
  if (coll == kTreeAllReduce) return tree_instance_by_op<I8, true>(op, proto, small);
  if (coll == kReduceScatter) return ring_instance_by_op<I8, kReduceScatter, true>(op, proto, small);
  return ring_instance_by_op<I8, kAllReduce, true>(op, proto, small);
}

}  // namespace ringar
