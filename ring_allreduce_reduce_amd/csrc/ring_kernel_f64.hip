// Ring AllReduce kernels for one element type (one translation unit per type
// so the instances compile in parallel).
#include "ring_kernel_impl.h"

namespace ringar {

template <int OP>
static const void* by_proto_f64(int proto) {
  if (proto == kLL) return (const void*)&ring_allreduce_kernel<F64, OP, kLL>;
  if (proto == kLL128) return (const void*)&ring_allreduce_kernel<F64, OP, kLL128>;
  return (const void*)&ring_allreduce_kernel<F64, OP, kSimple>;
}

const void* kernel_for_f64(int op, int proto) {
  switch (op) {
    case 0: return by_proto_f64<0>(proto);
    case 1: return by_proto_f64<1>(proto);
    case 2: return by_proto_f64<2>(proto);
    default: return by_proto_f64<3>(proto);
  }
}

}  // namespace ringar
