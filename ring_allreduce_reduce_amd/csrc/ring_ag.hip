// Ring AllGather kernels, eager form: a byte copy, so one instance per
// protocol (the host passes sizes in bytes).
#include "ring_instances.h"

namespace ringar {

const void* kernel_ag_for(int proto, bool small) { return ring_instance<I8, kAllGather, 0, false>(proto, small); }

}  // namespace ringar
