// Host-callable entry points of ring_kernel.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "ring_geometry.h"

namespace ringar {

// Kernel instance for (launch kind, dtype code, op code, protocol) of the
// public header (AllGather: a byte copy, dtype and op ignored); `small`: the
// form for lane parts of at most 1 KiB in 16-byte aligned buffers (LL and
// Simple only; ignored for LL128); `cap`: the captured form (ring AllReduce
// only).
const void* kernel_for(int coll, int dtype, int op, int proto, bool small, bool cap);

hipError_t launch_ring(int coll, int dtype, int op, int proto, bool small, bool cap, const KernelArgs& args,
                       int grid, int block, hipStream_t stream);

// Tree AllReduce launch (kernel_for(kTreeAllReduce, ...)).
hipError_t launch_tree(int dtype, int op, int proto, bool small, bool cap, const TreeArgs& args, int grid, int block,
                       hipStream_t stream);

hipError_t max_active_blocks(int coll, int dtype, int op, int proto, bool small, bool cap, int block, int* per_cu);

// Stream-ordered fill of `words` 64-bit words.
hipError_t launch_fill(uint64_t* p, uint64_t words, uint64_t value, hipStream_t stream);

}  // namespace ringar
