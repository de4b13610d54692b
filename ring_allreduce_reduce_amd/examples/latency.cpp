// Small-call latency of the C-ABI, measured from C: each case enqueues 2000
// back-to-back AllReduce calls of 8 virtual ranks (fp32 sum) on one stream
// and reports the device time per call (HIP events around the loop) and the
// host time to enqueue one call.  With the host faster than the device the
// first is the device-bound rate, free of any binding's per-call overhead.
// Each case is also captured into a HIP graph (the 2000 calls) and the
// graph's replay is timed the same way.
//
// Build (from the repository root, after the library is built):
//   hipcc -O2 -I include -o /tmp/ringar_latency ring_allreduce_reduce_amd/examples/latency.cpp \
//         -L ring_allreduce_reduce_amd -lringar -Wl,-rpath,$PWD/ring_allreduce_reduce_amd
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <vector>

#include "ringar.h"

#define CHECK_HIP(x)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

int main() {
  const int n = 8;
  const size_t max_count = 1 << 20;
  std::vector<void*> send(n), recv(n);
  for (int i = 0; i < n; i++) {
    CHECK_HIP(hipMalloc(&send[i], max_count * 4));
    CHECK_HIP(hipMalloc(&recv[i], max_count * 4));
    CHECK_HIP(hipMemset(send[i], 0, max_count * 4));
  }
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  struct Case {
    size_t count;
    ringar_algo_t algo;
    ringar_proto_t proto;
    const char* name;
  } cases[] = {{2, RINGAR_ALGO_RING, RINGAR_PROTO_LL, "ring LL 8 B"},
               {2, RINGAR_ALGO_TREE, RINGAR_PROTO_LL, "tree LL 8 B"},
               {2, RINGAR_ALGO_RING, RINGAR_PROTO_SIMPLE, "ring Simple 8 B"},
               {2, RINGAR_ALGO_RING, RINGAR_PROTO_LL128, "ring LL128 8 B"},
               {2048, RINGAR_ALGO_RING, RINGAR_PROTO_LL, "ring LL 8 KiB"},
               {8192, RINGAR_ALGO_TREE, RINGAR_PROTO_LL, "tree LL 32 KiB"},
               {65536, RINGAR_ALGO_TREE, RINGAR_PROTO_SIMPLE, "tree Simple 256 KiB"},
               {262144, RINGAR_ALGO_RING, RINGAR_PROTO_SIMPLE, "ring Simple 1 MiB"},
               {2, RINGAR_ALGO_AUTO, RINGAR_PROTO_AUTO, "auto 8 B"},
               {262144, RINGAR_ALGO_AUTO, RINGAR_PROTO_AUTO, "auto 1 MiB"}};
  const int calls = 2000;
  for (const Case& c : cases) {
    ringar_config_t cfg = {};
    cfg.skip_rank = -1;
    cfg.algo = c.algo;
    for (int k = 0; k < 20; k++) {
      ringar_result_t r = ringar_allreduce_ex(send.data(), recv.data(), c.count, RINGAR_FLOAT32, RINGAR_SUM, n, 0,
                                              c.proto, stream, &cfg);
      if (r != RINGAR_SUCCESS) {
        std::printf("%s: %s\n", c.name, ringar_result_string(r));
        return 1;
      }
    }
    CHECK_HIP(hipStreamSynchronize(stream));
    hipEvent_t start, stop;
    CHECK_HIP(hipEventCreate(&start));
    CHECK_HIP(hipEventCreate(&stop));
    const auto h0 = std::chrono::steady_clock::now();
    CHECK_HIP(hipEventRecord(start, stream));
    for (int k = 0; k < calls; k++)
      ringar_allreduce_ex(send.data(), recv.data(), c.count, RINGAR_FLOAT32, RINGAR_SUM, n, 0, c.proto, stream, &cfg);
    const auto h1 = std::chrono::steady_clock::now();
    CHECK_HIP(hipEventRecord(stop, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    float ms = 0;
    CHECK_HIP(hipEventElapsedTime(&ms, start, stop));
    const double host_us = std::chrono::duration<double, std::micro>(h1 - h0).count() / calls;
    const ringar_result_t err = ringar_get_async_error(stream);
    std::printf("%-22s device %6.2f us per call, host enqueue %5.2f us per call%s", c.name, ms * 1e3 / calls,
                host_us, err == RINGAR_SUCCESS ? "" : " (async error)");
    if (err != RINGAR_SUCCESS) return 1;
    {
      // the same calls captured into a graph, then one replay of it
      hipGraph_t graph;
      hipGraphExec_t exec;
      CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
      ringar_result_t cr = RINGAR_SUCCESS;
      for (int k = 0; k < calls && cr == RINGAR_SUCCESS; k++)
        cr = ringar_allreduce_ex(send.data(), recv.data(), c.count, RINGAR_FLOAT32, RINGAR_SUM, n, 0, c.proto, stream,
                                 &cfg);
      CHECK_HIP(hipStreamEndCapture(stream, &graph));
      if (cr != RINGAR_SUCCESS) {
        std::printf("\n%s under capture: %s\n", c.name, ringar_result_string(cr));
        return 1;
      }
      CHECK_HIP(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
      CHECK_HIP(hipGraphLaunch(exec, stream));   // first replay: warm
      CHECK_HIP(hipStreamSynchronize(stream));
      CHECK_HIP(hipEventRecord(start, stream));
      CHECK_HIP(hipGraphLaunch(exec, stream));
      CHECK_HIP(hipEventRecord(stop, stream));
      CHECK_HIP(hipStreamSynchronize(stream));
      CHECK_HIP(hipEventElapsedTime(&ms, start, stop));
      if (ringar_get_async_error(stream) != RINGAR_SUCCESS) {
        std::printf("\n%s: async error in the graph\n", c.name);
        return 1;
      }
      std::printf(", graph replay %6.2f us per call", ms * 1e3 / calls);
      CHECK_HIP(hipGraphExecDestroy(exec));
      CHECK_HIP(hipGraphDestroy(graph));
    }
    std::printf("\n");
    CHECK_HIP(hipEventDestroy(start));
    CHECK_HIP(hipEventDestroy(stop));
  }
  return 0;
}
