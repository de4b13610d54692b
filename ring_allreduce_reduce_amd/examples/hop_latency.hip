// One-hop latency between workgroups of one launch, within one XCD and
// across XCDs: a token goes round a ring of n single-wavefront workgroups,
// each waiting for its predecessor's store and then storing to its
// successor, with the device-scope accesses the library's flags use.  Rank r
// runs in workgroup r * stride; the other workgroups exit at once.  MI355X
// dispatches workgroups round-robin over its 8 XCDs, so stride 1 puts
// neighbouring ranks on different XCDs and stride 8 puts every rank on one.
// Two kinds of token: a 4-byte flag (a counter, as Simple's tail) and an
// 8-byte line {data, flag} stored and polled whole (as LL's lines).
//
// Build and run (from the repository root):
//   hipcc -O2 --offload-arch=gfx950 -o /tmp/hop_latency ring_allreduce_reduce_amd/examples/hop_latency.hip \
//         && /tmp/hop_latency
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

constexpr int kSlotWords = 64;   // one token per 256-byte line pair

// kind 0: 4-byte flag; kind 1: 8-byte line, flag in the high half.  Every
// wait gives up after spin_max polls (and then stops every rank), so the
// launch always ends.
__global__ void token_ring(uint32_t* slots, int n, int rounds, int stride, int kind, uint64_t* out,
                           uint32_t* gave_up, uint64_t spin_max) {
  if ((int)blockIdx.x % stride != 0) return;
  const int r = blockIdx.x / stride;
  if (r >= n || threadIdx.x != 0) return;
  uint32_t* mine = slots + r * kSlotWords;
  uint32_t* next = slots + ((r + 1) % n) * kSlotWords;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int k = 0; k < rounds; ++k) {
    if (!(r == 0 && k == 0)) {
      const uint32_t want = (uint32_t)(k * n + r);
      uint64_t spins = 0;
      while (true) {
        uint32_t flag;
        if (kind == 0) {
          flag = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const uint64_t line = __hip_atomic_load((uint64_t*)mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          flag = (uint32_t)(line >> 32);
        }
        if (flag == want) break;
        if (++spins > spin_max ||
            ((spins & 1023) == 0 && __hip_atomic_load(gave_up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
          __hip_atomic_store(gave_up, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
      }
    }
    const uint32_t f = (uint32_t)(k * n + r + 1);
    if (kind == 0)
      __hip_atomic_store(next, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store((uint64_t*)next, ((uint64_t)f << 32) | (uint32_t)k, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  if (r == 0) {
    out[0] = t0;
    out[1] = __builtin_amdgcn_s_memrealtime();
  }
}

int main() {
  const int n = 8, rounds = 2000;
  uint32_t* slots;
  uint64_t* out;
  uint32_t* gave_up;
  CHECK_HIP(hipMalloc(&slots, n * kSlotWords * sizeof(uint32_t)));
  CHECK_HIP(hipMalloc(&out, 2 * sizeof(uint64_t)));
  CHECK_HIP(hipMalloc(&gave_up, sizeof(uint32_t)));
  for (int kind = 0; kind < 2; ++kind)
    for (int rep = 0; rep < 3; ++rep)
      for (int stride : {1, 8}) {
        CHECK_HIP(hipMemset(slots, 0, n * kSlotWords * sizeof(uint32_t)));
        CHECK_HIP(hipMemset(gave_up, 0, sizeof(uint32_t)));
        CHECK_HIP(hipMemset(out, 0, 2 * sizeof(uint64_t)));
        CHECK_HIP(hipDeviceSynchronize());
        // at most 64 workgroups of 64 threads: all resident at once
        hipLaunchKernelGGL(token_ring, dim3(n * stride), dim3(64), 0, 0, slots, n, rounds, stride, kind, out,
                           gave_up, (uint64_t)1 << 20);
        CHECK_HIP(hipGetLastError());
        CHECK_HIP(hipDeviceSynchronize());
        uint64_t h[2];
        uint32_t g;
        CHECK_HIP(hipMemcpy(h, out, sizeof(h), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(&g, gave_up, sizeof(g), hipMemcpyDeviceToHost));
        if (g) {
          std::printf("a wait gave up\n");
          return 1;
        }
        // s_memrealtime counts at 100 MHz
        std::printf("%-12s %-14s %.3f us per hop (%d hops)\n", kind ? "8-byte line" : "4-byte flag",
                    stride == 8 ? "within an XCD" : "across XCDs", (h[1] - h[0]) / 100.0 / (rounds * n),
                    rounds * n);
        std::fflush(stdout);
      }
  return 0;
}
