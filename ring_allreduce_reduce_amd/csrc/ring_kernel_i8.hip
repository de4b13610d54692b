// Ring AllReduce kernels for one element type (one translation unit per type
// so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP>
static const void* by_proto_i8(int proto) {
  if (proto == kLL) return (const void*)&ring_allreduce_kernel<I8, OP, kLL>;
  if (proto == kLL128) return (const void*)&ring_allreduce_kernel<I8, OP, kLL128>;
  return (const void*)&ring_allreduce_kernel<I8, OP, kSimple>;
}

const void* kernel_for_i8(int op, int proto) {
  switch (op) {
    case 0: return by_proto_i8<0>(proto);
    case 1: return by_proto_i8<1>(proto);
    case 2: return by_proto_i8<2>(proto);
    default: return by_proto_i8<3>(proto);
  }
}

}  // namespace ringar
