// Tree AllReduce kernels for one element type, eager form (one translation
// unit per type so the instances compile in parallel).
#include "ring_instances.h"

namespace ringar {

const void* kernel_tree_for_f32(int op, int proto, bool small) {
  return tree_instance_by_op<F32, false>(op, proto, small);
}

}  // namespace ringar

#ifdef RINGAR_ROLE_PROFILE
// Reads the role profile of the last fp32 tree launch (a diagnostic build
// only: built with -DRINGAR_ROLE_PROFILE, see the role profile example).
extern "C" int ringar_role_profile(void* host, size_t bytes, int clear) {
  if (clear) {
    static unsigned long long zero[ringar::kRoleProfileWaves][8];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(ringar::g_role_profile), zero, sizeof(zero), 0,
                                  hipMemcpyHostToDevice);
  }
  if (bytes > sizeof(ringar::g_role_profile)) bytes = sizeof(ringar::g_role_profile);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(ringar::g_role_profile), bytes, 0, hipMemcpyDeviceToHost);
}
#endif
