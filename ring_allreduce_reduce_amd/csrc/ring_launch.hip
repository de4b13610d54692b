// Kernel dispatch by (launch kind, dtype, op, protocol, form), occupancy query and the fill
// kernel that clears FIFO memory and counters.
#include <hip/hip_runtime.h>

#include "ring_geometry.h"
#include "ring_kernel.h"

namespace ringar {

const void* kernel_for_i8(int op, int proto, bool small);
const void* kernel_for_i32(int op, int proto, bool small);
const void* kernel_for_f16(int op, int proto, bool small);
const void* kernel_for_bf16(int op, int proto, bool small);
const void* kernel_for_f32(int op, int proto, bool small);
const void* kernel_for_f64(int op, int proto, bool small);
const void* kernel_rs_for_i8(int op, int proto, bool small);
const void* kernel_rs_for_i32(int op, int proto, bool small);
const void* kernel_rs_for_f16(int op, int proto, bool small);
const void* kernel_rs_for_bf16(int op, int proto, bool small);
const void* kernel_rs_for_f32(int op, int proto, bool small);
const void* kernel_rs_for_f64(int op, int proto, bool small);
const void* kernel_ag_for(int proto, bool small);
const void* kernel_tree_for_i8(int op, int proto, bool small);
const void* kernel_tree_for_i32(int op, int proto, bool small);
const void* kernel_tree_for_f16(int op, int proto, bool small);
const void* kernel_tree_for_bf16(int op, int proto, bool small);
const void* kernel_tree_for_f32(int op, int proto, bool small);
const void* kernel_tree_for_f64(int op, int proto, bool small);
const void* kernel_captured_for_i8(int coll, int op, int proto, bool small);
const void* kernel_captured_for_i32(int coll, int op, int proto, bool small);
const void* kernel_captured_for_f16(int coll, int op, int proto, bool small);
const void* kernel_captured_for_bf16(int coll, int op, int proto, bool small);
const void* kernel_captured_for_f32(int coll, int op, int proto, bool small);
const void* kernel_captured_for_f64(int coll, int op, int proto, bool small);

// cap: the captured form (stream capture), whose instances sit in
// translation units of their own
const void* kernel_for(int coll, int dtype, int op, int proto, bool small, bool cap) {
  small = small && proto != kLL128;
  if (cap) {
    switch (coll == kAllGather ? 0 : dtype) {
      case 0: return kernel_captured_for_i8(coll, op, proto, small);
      case 1: return kernel_captured_for_i32(coll, op, proto, small);
      case 2: return kernel_captured_for_f16(coll, op, proto, small);
      case 3: return kernel_captured_for_bf16(coll, op, proto, small);
      case 4: return kernel_captured_for_f32(coll, op, proto, small);
      default: return kernel_captured_for_f64(coll, op, proto, small);
    }
  }
  if (coll == kAllGather) return kernel_ag_for(proto, small);
  if (coll == kTreeAllReduce) {
    switch (dtype) {
      case 0: return kernel_tree_for_i8(op, proto, small);
      case 1: return kernel_tree_for_i32(op, proto, small);
      case 2: return kernel_tree_for_f16(op, proto, small);
      case 3: return kernel_tree_for_bf16(op, proto, small);
      case 4: return kernel_tree_for_f32(op, proto, small);
      default: return kernel_tree_for_f64(op, proto, small);
    }
  }
  if (coll == kReduceScatter) {
    switch (dtype) {
      case 0: return kernel_rs_for_i8(op, proto, small);
      case 1: return kernel_rs_for_i32(op, proto, small);
      case 2: return kernel_rs_for_f16(op, proto, small);
      case 3: return kernel_rs_for_bf16(op, proto, small);
      case 4: return kernel_rs_for_f32(op, proto, small);
      default: return kernel_rs_for_f64(op, proto, small);
    }
  }
  switch (dtype) {
    case 0: return kernel_for_i8(op, proto, small);
    case 1: return kernel_for_i32(op, proto, small);
    case 2: return kernel_for_f16(op, proto, small);
    case 3: return kernel_for_bf16(op, proto, small);
    case 4: return kernel_for_f32(op, proto, small);
    default: return kernel_for_f64(op, proto, small);
  }
}

hipError_t launch_ring(int coll, int dtype, int op, int proto, bool small, bool cap, const KernelArgs& args,
                       int grid, int block, hipStream_t stream) {
  void* params[] = {const_cast<KernelArgs*>(&args)};
  return hipLaunchKernel(kernel_for(coll, dtype, op, proto, small, cap), dim3(grid), dim3(block), params, 0,
                         stream);
}

hipError_t launch_tree(int dtype, int op, int proto, bool small, bool cap, const TreeArgs& args, int grid, int block,
                       hipStream_t stream) {
  void* params[] = {const_cast<TreeArgs*>(&args)};
  return hipLaunchKernel(kernel_for(kTreeAllReduce, dtype, op, proto, small, cap), dim3(grid), dim3(block), params,
                         0, stream);
}

hipError_t max_active_blocks(int coll, int dtype, int op, int proto, bool small, bool cap, int block, int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, kernel_for(coll, dtype, op, proto, small, cap),
                                                      block, 0);
}

// Writes `value` into `words` 64-bit words (plain vector stores).  A kernel,
// not a memset, so that a caller may capture it in a graph.
__global__ void fill_u64_kernel(uint64_t* p, uint64_t words, uint64_t value) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t launch_fill(uint64_t* p, uint64_t words, uint64_t value, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  uint64_t blocks = div_up(words, 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, words, value);
  return hipGetLastError();
}

}  // namespace ringar
