// A short, fixed sequence of small AllReduce calls (8 virtual ranks, fp32
// sum, 50 calls per case on one stream) for per-dispatch profiling: the
// counters and kernel trace of each case's calls.
//
// Build (from the repository root, after the library is built):
//   hipcc -O2 -I include -o /tmp/ringar_small_calls ring_allreduce_reduce_amd/examples/small_calls.cpp \
//         -L ring_allreduce_reduce_amd -lringar -Wl,-rpath,$PWD/ring_allreduce_reduce_amd
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#include "ringar.h"

int main() {
  const int n = 8;
  const size_t bytes = 1 << 16;
  std::vector<void*> send(n), recv(n);
  for (int i = 0; i < n; i++) {
    if (hipMalloc(&send[i], bytes) != hipSuccess || hipMalloc(&recv[i], bytes) != hipSuccess) return 1;
    if (hipMemset(send[i], 0, bytes) != hipSuccess) return 1;
  }
  hipStream_t st;
  if (hipStreamCreate(&st) != hipSuccess) return 1;
  struct Case {
    size_t count;
    ringar_algo_t algo;
    ringar_proto_t proto;
    const char* name;
  } cases[] = {{2, RINGAR_ALGO_RING, RINGAR_PROTO_LL, "ring LL 8 B"},
               {2, RINGAR_ALGO_TREE, RINGAR_PROTO_LL, "tree LL 8 B"},
               {2, RINGAR_ALGO_RING, RINGAR_PROTO_SIMPLE, "ring Simple 8 B"},
               {2048, RINGAR_ALGO_RING, RINGAR_PROTO_LL, "ring LL 8 KiB"}};
  for (const Case& c : cases) {
    ringar_config_t cfg = {};
    cfg.skip_rank = -1;
    cfg.algo = c.algo;
    for (int k = 0; k < 50; k++) {
      ringar_result_t r = ringar_allreduce_ex(send.data(), recv.data(), c.count, RINGAR_FLOAT32, RINGAR_SUM, n, 0,
                                              c.proto, st, &cfg);
      if (r != RINGAR_SUCCESS) {
        std::printf("%s: %s\n", c.name, ringar_result_string(r));
        return 1;
      }
    }
    if (hipStreamSynchronize(st) != hipSuccess) return 1;
    const ringar_result_t e = ringar_get_async_error(st);
    std::printf("%s: 50 calls, %s\n", c.name, ringar_result_string(e));
    std::fflush(stdout);
    if (e != RINGAR_SUCCESS) return 1;
  }
  return 0;
}
