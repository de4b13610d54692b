// C ABI of the ring AllReduce library: argument checks, the alpha-beta
// protocol model, the launch plan, per-stream FIFO memory and the launch.
//
// Page sources: [ARCH] arganzheng.life, "NCCL architecture: topology,
// channels, algorithms and protocols" (§六.4 channel count by size, §六.5 FIFO
// of 8 steps, §七.2 protocols, §八 tuning model, §九.1 argument checks);
// [BOOK] aireadcode.com, "NCCL Source Code Deep Dive" (§1.3 enqueue-only
// semantics; Japanese edition ch. 5 selection rule and ch. 6 count == 0 and
// one-rank early outs, error classes).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ringar.h"
#include "ring_geometry.h"
#include "ring_kernel.h"

using namespace ringar;

namespace {

thread_local std::string t_last_error;

ringar_result_t hip_fail(hipError_t e, const char* what) {
  t_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return RINGAR_ERR_DEVICE;
}

#define HIP_TRY(call)                                   \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return hip_fail(e_, #call);   \
  } while (0)

size_t elem_size(int dtype) {
  static const size_t sz[] = {1, 4, 2, 2, 4, 8};
  return (dtype >= 0 && dtype <= 5) ? sz[dtype] : 0;
}

const char* kProtoName[3] = {"LL", "LL128", "Simple"};
const char* kDtypeName[6] = {"int8", "int32", "float16", "bfloat16", "float32", "float64"};
const char* kOpName[5] = {"sum", "prod", "min", "max", "avg"};
const char* kCollName[4] = {"AllReduce", "ReduceScatter", "AllGather", "Tree AllReduce"};

// ---------------------------------------------------------------- env
// RINGAR_* variables, each read once ([BOOK] §3.5: a parameter is read from
// the environment on first use and cached).
struct Env {
  int debug = 0;
  int proto_mask = 7;          // protocols AUTO may pick (bit p = protocol p)
  int algo_mask = 3;           // algorithms AUTO may pick (bit a = ringar_algo_t a)
  size_t chunk_bytes = 0;
  int max_nchannels = 0;
  uint32_t spin_limit_ms = 2000;
  int lanes = 0;
  int fifo_depth = 0;
  int block_map = 0;           // as ringar_config_t::block_map (a config's nonzero value wins)
  int tree_split = 1;          // 0: the tree's Simple roles never split
};

// RINGAR_PROTO / RINGAR_ALGO: comma-separated names (case-insensitive); a
// leading '^' excludes the listed ones instead ([ARCH] §八.5 NCCL_PROTO /
// NCCL_ALGO grammar, reduced to one list without per-function groups).
// names[i] sets bit i; an empty result means all.
int parse_name_list(const char* s, const char* const* names, int count) {
  const int all = (1 << count) - 1;
  if (!s || !*s) return all;
  bool exclude = false;
  if (*s == '^') { exclude = true; s++; }
  int mask = 0;
  std::string tok;
  auto flush = [&]() {
    std::string t;
    for (char ch : tok) t += (char)tolower((unsigned char)ch);
    for (int i = 0; i < count; i++)
      if (t == names[i]) mask |= 1 << i;
    tok.clear();
  };
  for (; *s; s++) {
    if (*s == ',') flush();
    else if (!isspace((unsigned char)*s)) tok += *s;
  }
  flush();
  int m = exclude ? (all & ~mask) : mask;
  return m ? m : all;
}

const char* const kProtoKeys[3] = {"ll", "ll128", "simple"};
const char* const kAlgoKeys[2] = {"ring", "tree"};

const Env& env() {
  static Env e;
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char* v = getenv("RINGAR_DEBUG")) e.debug = atoi(v);
    e.proto_mask = parse_name_list(getenv("RINGAR_PROTO"), kProtoKeys, 3);
    e.algo_mask = parse_name_list(getenv("RINGAR_ALGO"), kAlgoKeys, 2);
    if (const char* v = getenv("RINGAR_CHUNK_BYTES")) e.chunk_bytes = strtoull(v, nullptr, 0);
    if (const char* v = getenv("RINGAR_MAX_NCHANNELS")) e.max_nchannels = atoi(v);
    if (const char* v = getenv("RINGAR_SPIN_LIMIT_MS")) e.spin_limit_ms = (uint32_t)strtoul(v, nullptr, 0);
    if (const char* v = getenv("RINGAR_LANES")) e.lanes = atoi(v);
    if (const char* v = getenv("RINGAR_FIFO_DEPTH")) e.fifo_depth = atoi(v);
    if (const char* v = getenv("RINGAR_BLOCK_MAP")) e.block_map = atoi(v);
    if (const char* v = getenv("RINGAR_TREE_SPLIT")) e.tree_split = atoi(v);
  });
  return e;
}

// ---------------------------------------------------------------- model
// Built-in MI355X model.  The protocol efficiencies are the values the
// pages give (LL 0.5, LL128 about 0.94, Simple 1.0).  Latencies are fitted to
// small calls at n = 2..8 (T = base + 2(n-1) x step), bandwidths to 32-channel
// calls of 64-256 MiB per rank, both measured with this library on MI355X by
// `python -m ring_allreduce_reduce_amd.calibrate` (which also fits the Tree
// rows below).
// A channel of a small call runs one 64-thread wavefront per rank, hence 64
// threads per channel in the size rule.
ringar_model_t default_model() {
  ringar_model_t m;
  memset(&m, 0, sizeof(m));
  m.bw_per_channel = 10.279;
  m.ll_max_bw = 147.03;
  m.ll128_per_channel_max_bw = 8.554;
  m.eff[0] = 0.5; m.eff[1] = 0.94; m.eff[2] = 1.0;
  m.base_lat_us[0] = 4.93; m.base_lat_us[1] = 5.09; m.base_lat_us[2] = 4.93;
  m.hw_lat_us[0] = 1.188; m.hw_lat_us[1] = 2.44; m.hw_lat_us[2] = 1.331;
  m.max_channels = 32;
  m.max_pairs = 256;
  m.threads[0] = 64; m.threads[1] = 64; m.threads[2] = 64;
  m.thread_threshold[0] = 8; m.thread_threshold[1] = 8; m.thread_threshold[2] = 64;
  m.default_chunk_bytes[0] = 32768;
  m.default_chunk_bytes[1] = 491520;
  m.default_chunk_bytes[2] = 524288;
  // Tree rows: the pages' form with MI355X constants fitted the same way
  // (latency over n = 2..16 as base + 2 floor(log2 n) x step per level;
  // Simple bandwidth at 2 MiB per rank, LL at 1 MiB, LL128 at 8 MiB, where
  // tree and ring compete).  The ring's Simple bandwidth is that of the
  // direct form, which runs when the model takes Simple on the ring.
  m.tree_allreduce_eff = 0.5419;
  m.tree_per_channel_max_bw = 1e9;
  m.tree_ll_divisor = 1.7201;
  m.tree_ll128_factor = 0.877;
  m.tree_ll128_per_channel_max_bw = 1e9;
  m.tree_base_lat_us[0] = 5.63; m.tree_base_lat_us[1] = 4.81; m.tree_base_lat_us[2] = 5.69;
  m.tree_hw_lat_us[0] = 1.235; m.tree_hw_lat_us[1] = 3.506; m.tree_hw_lat_us[2] = 1.696;
  m.tree_correction = 0;
  return m;
}

// Bandwidth correction of the Tree AllReduce by message size, per protocol,
// indexed by floor(log2(bytes / 64)) ([BOOK] Japanese edition ch. 5 §四: the
// pages' table, measured on NVIDIA systems; used only when a model sets
// tree_correction).
const float kTreeCorrection[3][24] = {
    {1.0f, 1.0f, 1.0f, 1.0f, .9f, .8f, .7f, .7f, .7f, .7f, .6f, .5f, .4f, .4f, .5f, .6f, .7f, .8f, .9f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f},
    {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, .9f, .8f, .8f, .8f, .7f, .6f, .6f, .6f, .6f, .6f, .6f, .8f, .9f, .9f, .9f, .9f, 1.0f, 1.0f, 1.0f},
    {.9f, .9f, .9f, .9f, .9f, .9f, .9f, .8f, .7f, .6f, .6f, .5f, .5f, .5f, .5f, .6f, .7f, .8f, .7f, .7f, .8f, .9f, .9f, .9f}};

int floor_log2(uint64_t x) {
  int r = -1;
  while (x) { x >>= 1; r++; }
  return r;
}

// Bus bandwidth of protocol p on nch channels ([ARCH] §八.1).
double bus_bw(const ringar_model_t& m, int nch, int p) {
  double bus = nch * m.bw_per_channel;
  if (p == kLL) return std::min(m.ll_max_bw, bus * m.eff[0]);
  if (p == kLL128) return std::min(bus * m.eff[1], nch * m.ll128_per_channel_max_bw);
  return bus * m.eff[2];
}

// Predicted microseconds of one call ([ARCH] §八.1-八.2):
// base + nsteps step latencies + bytes / (1000 x bus bandwidth x n / nsteps),
// with nsteps = 2(n-1) for the AllReduce and n-1 for its halves, whose
// `bytes` count the whole n-block buffer (the tuning model's rule).
double predict_us(const ringar_model_t& m, int n, int nch, int p, size_t bytes, int coll = kAllReduce) {
  double nsteps = (coll == kAllReduce ? 2.0 : 1.0) * (n - 1);
  double alg = bus_bw(m, nch, p) * n / nsteps;
  double lat = m.base_lat_us[p] + nsteps * m.hw_lat_us[p];
  return lat + (double)bytes / (1000.0 * alg);
}

// Tree AllReduce bus bandwidth of protocol p on nch channels ([BOOK]
// Japanese edition ch. 5 §四).
double tree_bus_bw(const ringar_model_t& m, int nch, int p) {
  double bus = std::min(nch * m.bw_per_channel * m.tree_allreduce_eff, nch * m.tree_per_channel_max_bw);
  if (p == kLL) bus = std::min(bus / m.tree_ll_divisor, m.ll_max_bw);
  else if (p == kLL128) bus = std::min(bus * m.tree_ll128_factor, nch * m.tree_ll128_per_channel_max_bw);
  return bus;
}

// Predicted microseconds of one tree AllReduce: every rank is one vertex, so
// the tree's depth term is 2 x floor(log2 n) steps; algorithm bandwidth =
// bus bandwidth x 0.5, corrected by size when the model asks for it.
double predict_tree_us(const ringar_model_t& m, int n, int nch, int p, size_t bytes) {
  double alg = tree_bus_bw(m, nch, p) * 0.5;
  const int ls = floor_log2((uint64_t)bytes >> 6);
  if (m.tree_correction && ls >= 0 && ls < 23) alg *= kTreeCorrection[p][ls];
  double lat = m.tree_base_lat_us[p] + 2.0 * floor_log2((uint64_t)n) * m.tree_hw_lat_us[p];
  return lat + (double)bytes / (1000.0 * alg);
}

// Fastest enabled (algorithm, protocol) of an AllReduce.  Candidates are
// numbered Tree LL, LL128, Simple, Ring LL, LL128, Simple (the pages' model
// map) and visited from the last, replaced only on a strictly smaller time.
// times6 receives the six times in that order.  Returns false when nothing
// is enabled.
bool select_algo_proto(const ringar_model_t& m, int n, int nch, size_t bytes, int algo_mask, int proto_mask,
                       int* algo, int* proto, double* times6) {
  double t[6];
  for (int p = 0; p < 3; p++) {
    t[p] = predict_tree_us(m, n, nch, p, bytes);
    t[3 + p] = predict_us(m, n, nch, p, bytes);
  }
  if (times6) memcpy(times6, t, sizeof(t));
  double best_t = INFINITY;
  bool found = false;
  for (int id = 5; id >= 0; id--) {
    const int a = id >= 3 ? RINGAR_ALGO_RING : RINGAR_ALGO_TREE, p = id % 3;
    if (!(algo_mask & (1 << a)) || !(proto_mask & (1 << p))) continue;
    if (t[id] < best_t) {
      best_t = t[id];
      *algo = a;
      *proto = p;
      found = true;
    }
  }
  return found;
}

// The binary tree of [ARCH] §五.4 over ranks 0..n-1: a rank's lowest set bit
// b decides its level; its parent clears b and sets the bit above (or only
// clears b when that rank does not exist); its children are rank - b/2 and
// the largest rank + b/2^k (k >= 1) that exists.  Rank 0 is the root with the
// single child B/2, B = the smallest power of two >= n.  The second tree
// mirrors ranks (r -> n-1-r) for even n and shifts them by one for odd n.
// Child slots keep their order through the renaming.
void tree_links(int n, int t, int rank, int* up, int* c0, int* c1) {
  int r = rank;
  if (t == 1) r = (n % 2 == 0) ? n - 1 - rank : (rank + n - 1) % n;
  int b = 1;
  while (b < n && !(r & b)) b <<= 1;
  int u, d0, d1;
  if (r == 0) {
    u = -1;
    d0 = -1;
    d1 = n > 1 ? b >> 1 : -1;
  } else {
    u = (r ^ b) | (b << 1);
    if (u >= n) u = r ^ b;
    d0 = (b >> 1) ? r - (b >> 1) : -1;
    d1 = -1;
    for (int h = b >> 1; h > 0; h >>= 1)
      if (r + h < n) { d1 = r + h; break; }
  }
  auto back = [&](int x) {
    if (x < 0 || t == 0) return x;
    return (n % 2 == 0) ? n - 1 - x : (x + 1) % n;
  };
  *up = back(u);
  *c0 = back(d0);
  *c1 = back(d1);
}

// The wavefronts of the split tree form per (channel, lane) on tree t, in
// vertex order (reduce role, then broadcast role; a split role twice, its
// halves 0 and 1), written to role_of as vertex | broadcast << 6 | half << 7.
int tree_split_roles(int n, int t, uint8_t* role_of) {
  int cnt = 0;
  for (int v = 0; v < n; v++) {
    int u, c0, c1;
    tree_links(n, t, v, &u, &c0, &c1);
    const int nk = (c0 >= 0 ? 1 : 0) + (c1 >= 0 ? 1 : 0);
    const int up = tree_role_splits(false, u < 0, nk) ? 2 : 1;
    for (int h = 0; h < up; h++) role_of[cnt++] = (uint8_t)(v | (h << 7));
    if (u >= 0) {
      const int down = tree_role_splits(true, false, nk) ? 2 : 1;
      for (int h = 0; h < down; h++) role_of[cnt++] = (uint8_t)(v | 64 | (h << 7));
    }
  }
  return cnt;
}

int model_max_channels(const ringar_model_t& m, int n) {
  int c = std::min(m.max_channels, m.max_pairs / std::max(1, n));
  return std::max(1, std::min(c, kMaxChannels));
}

// Fastest enabled protocol.  Candidates are visited Simple, LL128, LL (the
// pages' list is built by pushing to the front) and replaced only on a
// strictly smaller time, so ties go to Simple, then LL128.
int select_proto(const ringar_model_t& m, int n, int nch, size_t bytes, int mask, double* times,
                 int coll = kAllReduce) {
  int best = -1;
  double best_t = INFINITY;
  for (int p = 2; p >= 0; p--) {
    double t = predict_us(m, n, nch, p, bytes, coll);
    if (times) times[p] = t;
    if (!(mask & (1 << p))) continue;
    if (t < best_t) { best = p; best_t = t; }
  }
  return best;
}

// Fastest enabled protocol of three model times (the tie rule of
// select_proto); -1 when none is enabled.
int select_proto_of(const double* times, int mask) {
  int best = -1;
  double best_t = INFINITY;
  for (int p = 2; p >= 0; p--)
    if ((mask & (1 << p)) && times[p] < best_t) { best = p; best_t = times[p]; }
  return best;
}

// Channel count by size ([ARCH] §六.4): drop channels while each thread would
// get fewer than threshold bytes; LL's threshold is multiplied by n on a ring.
int auto_channels(const ringar_model_t& m, int n, int p, size_t bytes, int start, bool ring = true) {
  int nc = start;
  double thr = (double)m.thread_threshold[p] * (p == kLL && ring ? n : 1);
  while (nc > 1 && (double)bytes < (double)nc * m.threads[p] * thr) nc--;
  return nc;
}

// ---------------------------------------------------------------- plan
struct Plan {
  int kind = kAllReduce;   // launch kind (kTreeAllReduce for the tree)
  int proto = kSimple;
  int nch = 1;
  size_t chunk_bytes = 0;
  uint64_t chunk_elems = 0;
  uint64_t per_channel = 0;
  int lanes = 1;
  int depth = kMaxSteps;
  bool small = false;      // every lane part fits the small-slice form
  bool direct = false;     // direct form requested and possible (if out of place)
  bool direct_auto = false;// the library chose it (a captured call then keeps its FIFOs)
  bool tree_split = false; // the split tree form (tree_body_split)
  int tree_waves = 0;      // its wavefronts per (channel, lane)
  bool xcd_major = false;  // block ids map XCD-major (launch_grid, block_group)
  int lanes_per_block = 1;
  int grid = 0;
  int block = 64;
  uint64_t max_steps = 0;
  uint64_t conns = 0;      // FIFO connections of the launch
  double times[3] = {0, 0, 0};
  double tree_times[3] = {0, 0, 0};
  double ring_times[3] = {0, 0, 0};
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr uint64_t kTargetWaves = 4096;
constexpr uint64_t kTreeSplitMinChannelBytes = 256 << 10;   // the split tree form's smallest channel

// Largest bytes per rank that take the XCD-major block mapping (below).
constexpr uint64_t kXcdMajorMaxBytes = 512 << 10;
constexpr uint64_t kXcdMajorLL128MaxBytes = 32 << 10;
// Smallest bytes per rank for which the library itself takes the direct form.
constexpr uint64_t kDirectAutoMinBytes = 256 << 10;

// FIFO bytes that all connections of a call write in one step of every
// lane, summed over the FIFO depth, above which the depth is halved.  The
// FIFOs are written by one wavefront and read by another a step later; on
// MI355X they stream fastest while this footprint stays well inside the
// 256 MB Infinity Cache (64 MiB per rank over 16 channels: 436 us at depth
// 8 with 512 MiB in flight, 432 us at depth 2 with 128 MiB).
constexpr uint64_t kFifoBudgetBytes = 128ull << 20;
// LL128 runs fewer, longer lanes (below) and gains from the deeper FIFO up to
// twice that footprint (bf16, 8 lanes, 32 MiB per rank: depth 4 234 us, 136
// MiB in flight; 16 MiB depth 8 138 us against depth 4 137 us).
constexpr uint64_t kLL128FifoBudgetBytes = 256ull << 20;
constexpr uint64_t kLL128LaneBytes = 8192;
constexpr int kLL128MaxAutoLanes = 8;

// FIFO bytes that carry `bytes` of data in one slot of the protocol.
uint64_t fifo_bytes_for(int proto, uint64_t bytes) {
  if (proto == kSimple) return bytes;
  if (proto == kLL) return 2 * bytes;
  return div_up(bytes, (uint64_t)120) * 128;
}

// capacity_waves: wavefronts of this kernel the GPU holds at once (0 when no
// GPU is visible: then 4096 is assumed).
// coll: kAllReduce (count = elements per rank; the algorithm comes from the
// config) or one of its halves (count = elements per block; AllGather plans
// bytes, dtype int8).
ringar_result_t make_plan(int coll, size_t count, int dtype, int n, int nchannels, int proto,
                          const ringar_config_t* cfg, uint64_t capacity_waves, Plan* out,
                          bool captured = false) {
  const Env& E = env();
  const size_t es = elem_size(dtype);
  if (!es) return RINGAR_ERR_INVALID_ARGUMENT;
  if (n < 1 || n > kMaxRanks) return RINGAR_ERR_INVALID_ARGUMENT;
  if (nchannels < 0 || nchannels > kMaxChannels) return RINGAR_ERR_INVALID_ARGUMENT;
  if (proto < RINGAR_PROTO_AUTO || proto > RINGAR_PROTO_SIMPLE) return RINGAR_ERR_INVALID_ARGUMENT;
  const int algo_req = cfg ? cfg->algo : RINGAR_ALGO_RING;
  if (algo_req < RINGAR_ALGO_RING || algo_req > RINGAR_ALGO_AUTO) return RINGAR_ERR_INVALID_ARGUMENT;
  if (coll != kAllReduce && algo_req == RINGAR_ALGO_TREE) return RINGAR_ERR_INVALID_ARGUMENT;
  ringar_model_t dm = default_model();
  const ringar_model_t& m = (cfg && cfg->model) ? *cfg->model : dm;
  size_t chunk_bytes = (cfg && cfg->chunk_bytes) ? cfg->chunk_bytes : E.chunk_bytes;
  if (chunk_bytes % 16 != 0) return RINGAR_ERR_INVALID_ARGUMENT;
  int lanes = (cfg && cfg->lanes) ? cfg->lanes : E.lanes;
  if (lanes && (!is_pow2(lanes) || lanes > kMaxLanes)) return RINGAR_ERR_INVALID_ARGUMENT;
  const int depth = (cfg && cfg->fifo_depth) ? cfg->fifo_depth : E.fifo_depth;
  if (depth && (!is_pow2(depth) || depth < kMinSteps || depth > kMaxSteps)) return RINGAR_ERR_INVALID_ARGUMENT;

  Plan P;
  const bool halves = coll != kAllReduce;
  const size_t bytes = count * es * (halves ? (size_t)n : 1);
  int maxc = model_max_channels(m, n);
  if (E.max_nchannels > 0) maxc = std::min(maxc, E.max_nchannels);
  const int model_nch = nchannels > 0 ? nchannels : maxc;
  int best = select_proto(m, n, model_nch, bytes, E.proto_mask, P.ring_times, coll);
  // Algorithm: the ring unless the config asks for the tree, or for the
  // model's choice (AllReduce only, more than one rank).
  bool tree = false;
  if (!halves && n > 1) {
    for (int p = 0; p < 3; p++) P.tree_times[p] = predict_tree_us(m, n, model_nch, p, bytes);
    if (algo_req == RINGAR_ALGO_TREE) {
      tree = true;
      best = select_proto_of(P.tree_times, E.proto_mask);
    } else if (algo_req == RINGAR_ALGO_AUTO) {
      int a = RINGAR_ALGO_RING, p = best;
      const int pmask = proto >= 0 ? (1 << proto) : E.proto_mask;
      if (select_algo_proto(m, n, model_nch, bytes, E.algo_mask, pmask, &a, &p, nullptr)) {
        tree = a == RINGAR_ALGO_TREE;
        best = p;
      }
    }
  }
  if (proto < 0 && best < 0 && n > 1) return RINGAR_ERR_INVALID_USAGE;
  P.kind = tree ? kTreeAllReduce : coll;
  memcpy(P.times, tree ? P.tree_times : P.ring_times, sizeof(P.times));
  P.proto = proto >= 0 ? proto : (n == 1 ? (int)kSimple : best);
  P.nch = nchannels > 0 ? nchannels : (n == 1 ? 1 : auto_channels(m, n, P.proto, bytes, maxc, !tree));
  P.per_channel = channel_len(count, P.nch, (uint32_t)es);
  P.chunk_bytes = chunk_bytes ? chunk_bytes : m.default_chunk_bytes[P.proto];
  // The split tree form (below) is wanted for eager Simple tree calls of at
  // least kTreeSplitMinChannelBytes per channel.
  const bool split_wanted = tree && P.proto == kSimple && !captured && E.tree_split && n > 1 &&
                            P.per_channel * es >= kTreeSplitMinChannelBytes;
  if (tree && !chunk_bytes) {
    // The tree moves a whole chunk up and then down, so a channel needs
    // several chunks for the two directions to overlap: a quarter of the
    // channel, kept between 8 KiB (4 KiB for LL) and 2 MiB / channels (at
    // least 64 KiB), so that all channels together keep about 2 MiB in
    // flight.  Measured on MI355X at n = 8, fp32: 32 channels, against
    // 512 KiB chunks, 2 MiB per rank 47.5 -> 37.9 us, 8 MiB 133.7 -> 99.4
    // us, 64 MiB 620 -> 534 us; at 64 MiB the best chunk is 64 KiB at 32
    // channels (529 us), 128 KiB at 16 (550 against 593 us at 64 KiB) and
    // 256 KiB at 8 (531 against 659 us).  The split form keeps twice that
    // in flight, in chunks of half the channel: at 64 MiB, 32 channels,
    // 128 KiB chunks take 483 us against 495 at 64 KiB; 8 MiB 83 against
    // 86 us; n = 5 318 against 351 us.
    const uint64_t lo = P.proto == kLL ? 4096 : 8192;
    const uint64_t in_flight = split_wanted ? (4u << 20) : (2u << 20);
    // (whole 16-byte units: channel counts that are not powers of two)
    const uint64_t hi = std::min<uint64_t>(
        std::max<uint64_t>(split_wanted ? 131072 : 65536, in_flight / (uint64_t)P.nch / 16 * 16), P.chunk_bytes);
    P.chunk_bytes = std::min(hi, std::max(lo, align_up(P.per_channel * es / (split_wanted ? 2 : 4), 16)));
  }
  if (P.chunk_bytes == 0 || P.chunk_bytes % 16 != 0 || P.chunk_bytes % es != 0)
    return RINGAR_ERR_INVALID_ARGUMENT;
  P.chunk_elems = P.chunk_bytes / es;

  // Lanes: wavefronts sharing each (rank, channel) chunk, each with its own
  // FIFO.  A primitive's part of a chunk may fill at most half the FIFO
  // (kMaxSlicesPerPart slots, like a chunk of NCCL_STEPS/2 steps): a
  // receiver keeps its slot until its own send is done, so parts of a full
  // FIFO's size would let every FIFO of the ring fill up and deadlock.
  // Beyond that, one lane per started KiB of chunk (a power of two, up to
  // 32), and at most
  // kTargetWaves wavefronts in all (on MI355X, 64 MiB over 16 channels: 32
  // lanes, 4096 wavefronts, ran 11% faster than 16 lanes) and never more
  // than the GPU holds at once (all of them wait on each other).  Lanes
  // change no result.
  // (The halves' loops take up to one chunk of every block, the tree's one
  // chunk of the channel.)
  const uint64_t first_chunk =
      (halves || tree) ? std::max<uint64_t>(1, std::min<uint64_t>(P.chunk_elems, P.per_channel))
      : P.per_channel >= (uint64_t)n * P.chunk_elems
          ? P.chunk_elems
          : align_up(div_up(std::max<uint64_t>(1, P.per_channel), (uint64_t)n), align_elems((uint32_t)es));
  const uint64_t slot = slot_elems(P.proto, (uint32_t)es);
  auto slices_for = [&](int L) { return div_up(lane_part(first_chunk, L, (uint32_t)es, P.proto), slot); };
  // wavefronts per lane: one per rank on the ring, 2n - 1 roles on the tree
  const uint64_t waves_per_lane = (uint64_t)(tree ? tree_roles(n) : n) * P.nch;
  const bool forced_lanes = lanes != 0;
  if (!forced_lanes) {
    const uint64_t want = std::max<uint64_t>(1, div_up(first_chunk * es, lane_gran_bytes(P.proto)));
    lanes = 1;
    while (lanes < (int)std::min<uint64_t>(want, kMaxLanes)) lanes *= 2;
    const uint64_t cap = std::min<uint64_t>(kTargetWaves, capacity_waves ? capacity_waves : 4096);
    while (lanes > 1 && waves_per_lane * lanes > cap && slices_for(lanes / 2) <= kMaxSlicesPerPart)
      lanes /= 2;
    while (lanes < kMaxLanes && slices_for(lanes) > kMaxSlicesPerPart) lanes *= 2;
  }
  // Automatic lane counts need not be powers of two (only whole workgroups
  // of 4): when a part needs more than one slice, take the smallest larger
  // multiple of 4 lanes that the GPU holds and that needs fewer slices; a
  // short trailing slice costs a whole flag round trip (bf16 LL128 at 64 MiB
  // per rank: 8 lanes of 32 KiB parts need a 30 KiB and a 2 KiB slice each,
  // 12 lanes need one).
  // LL128 on the ring takes its own rule below.
  const bool ll128_ring = P.proto == kLL128 && !tree;
  if (!forced_lanes && !ll128_ring && lanes >= 4 && slices_for(lanes) > 1) {
    const uint64_t cap = std::min<uint64_t>(kTargetWaves, capacity_waves ? capacity_waves : 4096);
    for (int L = lanes + 4; L <= kMaxLanes && waves_per_lane * L <= cap; L += 4)
      if (slices_for(L) < slices_for(lanes)) {
        lanes = L;
        break;
      }
  }
  // The slices stream whole groups without per-lane conditions (Simple:
  // 64 x 8 packets = 8 KiB; LL128: 32 lines = 3840 data bytes) and a
  // shorter remainder lane by lane.  When the parts above are shorter than
  // one group and the largest power of two of lanes whose part holds a whole
  // group is still at least 2, take it.  Measured at n = 8, 32 channels:
  // bf16 LL128 2 MiB per rank 8 -> 2 lanes 67.6 -> 54.6 us, 4 MiB 8 -> 4
  // lanes 95.6 -> 79.2 us; fp32 Simple 8 MiB 16 -> 4 lanes 68.1 -> 64.6 us,
  // 16 MiB 16 -> 8 lanes 118.5 -> 110.8 us.  A single lane was slower, and
  // Simple parts of the small-slice form (at most 1 KiB) keep their lanes.
  if (!forced_lanes && P.proto == kSimple && !tree &&
      lane_part(first_chunk, lanes, (uint32_t)es, P.proto) * es > kSmallSliceBytes) {
    int whole = 1;
    while ((uint64_t)(whole * 2) * kSimpleGroupBytes <= first_chunk * es) whole *= 2;
    if (whole >= 2 && whole < lanes) lanes = whole;
  }
  // LL128 on the ring (and its halves): a lane per 8 KiB of chunk, a power
  // of two between 2 and 8 (then more only if a part would need more than
  // half the FIFO).  Longer parts stream several 64-line row iterations per
  // flag round trip; more lanes than that only crowd the memory system.
  // Measured on MI355X, bf16 sum, n = 8, 32 channels, lanes / depth: 1 MiB
  // per rank 2 lanes 54 us against 8 lanes 64 us; 2 MiB 57 against 84 (16
  // lanes); 16 MiB 4 lanes 132 us; 32 MiB 8 lanes 234 against 256 (16); 64
  // MiB 8 lanes 456 against 468 (4) and 479 (16); fp32 at 128 MiB 8 lanes
  // 927 against 972 (16) and 939 (4).
  if (!forced_lanes && ll128_ring) {
    lanes = 2;
    while (lanes < kLL128MaxAutoLanes && (uint64_t)(lanes * 2) * kLL128LaneBytes <= first_chunk * es) lanes *= 2;
    while (lanes < kMaxLanes && slices_for(lanes) > kMaxSlicesPerPart) lanes *= 2;
  }
  // The split tree form (eager Simple calls of at least
  // kTreeSplitMinChannelBytes per channel): the roles that move four or more
  // units per element run as two wavefronts, so a lane takes more
  // wavefronts and the grid's 4096 fewer lanes, of any count (whole
  // workgroups of 4, 2 or 1 wavefronts).  Measured on MI355X (fp32, with
  // its chunk rule above, against one wavefront a role): 2-17% off calls of
  // 64 MiB per rank at n = 2..16; at 256 KiB per channel n = 2, 3 and 8 gain
  // 2-4% while n = 4 and 6 lose 5-8%; below 256 KiB per channel the fewer
  // lanes cost more than the halves gain (3-29% slower at n = 8).
  P.tree_split = false;
  if (split_wanted) {
    uint8_t roles[2][4 * kMaxRanks];
    const int r0 = tree_split_roles(n, 0, roles[0]), r1 = tree_split_roles(n, 1, roles[1]);
    const uint64_t wpl2 = (uint64_t)r0 * P.nch;
    const uint64_t cap = std::min<uint64_t>(kTargetWaves, capacity_waves ? capacity_waves : 4096);
    int l2 = lanes;
    if (!forced_lanes) {
      const uint64_t want = std::max<uint64_t>(1, div_up(first_chunk * es, lane_gran_bytes(P.proto)));
      l2 = (int)std::min<uint64_t>(std::min<uint64_t>(want, kMaxLanes), cap / wpl2);
    }
    const bool small_parts = l2 >= 1 && lane_part(first_chunk, l2, (uint32_t)es, P.proto) * es <= kSmallSliceBytes;
    if (r0 == r1 && l2 >= 1 && wpl2 * l2 <= cap && !small_parts && slices_for(l2) <= kMaxSlicesPerPart) {
      lanes = l2;
      P.tree_split = true;
      P.tree_waves = r0;
    }
  }
  // (one rank moves no FIFO slot: its call is a copy, whatever the knobs)
  if (n > 1 && slices_for(lanes) > kMaxSlicesPerPart)
    return forced_lanes ? RINGAR_ERR_INVALID_USAGE : RINGAR_ERR_INVALID_ARGUMENT;
  P.lanes = lanes;

  // FIFO depth: the deepest of 8, 4, 2 slots whose footprint fits
  // kFifoBudgetBytes, but always at least twice the slots of a part.
  const uint64_t waves = waves_per_lane * lanes;
  const uint64_t step_bytes =
      fifo_bytes_for(P.proto, std::min<uint64_t>(lane_part(first_chunk, lanes, (uint32_t)es, P.proto), slot) * es);
  if (depth) {
    if (n > 1 && (uint64_t)slices_for(lanes) > (uint64_t)depth / 2) return RINGAR_ERR_INVALID_USAGE;
    P.depth = depth;
  } else {
    P.depth = kMaxSteps;
    const uint64_t budget = P.proto == kLL128 ? kLL128FifoBudgetBytes : kFifoBudgetBytes;
    while (P.depth > kMinSteps && waves * P.depth * step_bytes > budget &&
           (uint64_t)slices_for(lanes) <= (uint64_t)P.depth / 4)
      P.depth /= 2;
  }
  // Lane parts of at most 1 KiB (one 16-byte packet per lane and step) run
  // the straight-line form of LL and Simple when the buffers are aligned.
  // The direct form: on request (direct = 1), or by the library's choice
  // (direct = 0) when the model chose the protocol and took Simple on the
  // ring for at least kDirectAutoMinBytes per rank.  Measured on MI355X, ring
  // Simple, automatic channels, FIFO against direct: n = 8 fp32 256 KiB
  // 27.0 / 26.1 us, 2 MiB 38.2 / 34.4, 8 MiB 64.6 / 53.6, 64 MiB 413 / 358,
  // 1 GiB 6531 / 5352; bf16 8 MiB 65.3 / 54.3; n = 16 fp32 64 MiB 852 / 756;
  // n = 4 fp32 8 MiB 33.4 / 33.8, 64 MiB 195 / 159.
  const int direct_req = cfg ? cfg->direct : 0;
  if (direct_req < 0 || direct_req > 2) return RINGAR_ERR_INVALID_ARGUMENT;
  const bool direct_ok = P.kind == kAllReduce && P.proto == kSimple && n > 1;
  P.direct_auto = direct_req == 0 && proto < 0 && direct_ok && (uint64_t)bytes >= kDirectAutoMinBytes;
  P.direct = direct_ok && (direct_req == 1 || P.direct_auto);
  P.small = P.proto != kLL128 && lane_part(first_chunk, lanes, (uint32_t)es, P.proto) * es <= kSmallSliceBytes &&
            !(cfg && cfg->force_general) && !P.direct;
  // whole workgroups: 4 lanes, else 2, else 1
  P.lanes_per_block = lanes % 4 == 0 ? 4 : lanes % 2 == 0 ? 2 : 1;
  P.block = 64 * P.lanes_per_block;
  const int groups = P.nch * (lanes / P.lanes_per_block);
  // Block mapping: latency-bound calls put every rank (tree: every role) of
  // a channel on one XCD, where a flag or tail store reaches its reader
  // sooner (a token passed round 8 single-wavefront workgroups, the example
  // hop_latency.hip: 0.32-0.54 us per hop within one XCD against 0.49-0.58 us
  // across XCDs, depending on the box).  Bandwidth-bound calls keep the
  // linear mapping, which spreads each channel's FIFO traffic over the XCDs.
  // Measured at n = 8, fp32 sum, automatic channels (HIP events per call):
  // XCD-major faster up to 512 KiB per rank (ring Simple 8 B 23.1 -> 17.5
  // us, tree LL 8 B 9.4 -> 8.4, tree Simple 512 KiB 21.7 -> 19.7), slower
  // from 2 MiB (ring LL 41.9 -> 54.1, tree Simple 8 MiB 87.5 -> 100.6), and
  // LL128 slower from 128 KiB (ring 36.8 -> 39.6).
  const uint64_t xcd_limit = P.proto == kLL128 ? kXcdMajorLL128MaxBytes : kXcdMajorMaxBytes;
  const int block_map = (cfg && cfg->block_map) ? cfg->block_map : E.block_map;
  if (block_map < 0 || block_map > 2) return RINGAR_ERR_INVALID_ARGUMENT;
  P.xcd_major = block_map ? block_map == 2 : (uint64_t)bytes <= xcd_limit;
  const int members = P.tree_split ? P.tree_waves : tree ? tree_roles(n) : n;
  P.grid = launch_grid(members, groups, P.xcd_major);
  // The XCD-major grid pads the groups to whole rounds of 8 so that every
  // XCD takes the same number of workgroups; the padded grid must still be
  // resident at once (workgroup b runs on XCD b mod 8, so a round that does
  // not fit stalls the dispatch).  By size, such a call takes the linear
  // mapping; a forced XCD-major mapping is refused.
  const uint64_t resident = std::min<uint64_t>(kTargetWaves, capacity_waves ? capacity_waves : 4096);
  if (P.xcd_major && (uint64_t)P.grid * P.lanes_per_block > resident) {
    if (block_map == 2) return RINGAR_ERR_INVALID_USAGE;
    P.xcd_major = false;
    P.grid = launch_grid(members, groups, false);
  }
  // A forced lane count whose grid the GPU cannot hold at once is refused
  // here, as the launch would refuse it (the kernel's residency is known
  // only with a device; without one the launch decides).
  if (forced_lanes && capacity_waves && (uint64_t)P.grid * P.lanes_per_block > capacity_waves)
    return RINGAR_ERR_INVALID_USAGE;
  P.conns = (uint64_t)P.nch * n * lanes * (tree ? 2 : 1);

  // Upper bound of FIFO steps any connection takes in this call.
  const uint64_t loops =
      std::max<uint64_t>(1, div_up(P.per_channel, ((halves || tree) ? 1 : (uint64_t)n) * P.chunk_elems));
  const uint64_t prims = tree ? 1 : (uint64_t)(halves ? n : 2 * n - 1);   // primitives per loop
  P.max_steps = loops * prims * (slices_for(lanes) + 1);
  *out = P;
  return RINGAR_SUCCESS;
}

// ---------------------------------------------------------------- resources
// FIFO memory, counters and the error word of one (device, stream).  All
// counters and flags are absolute step numbers below `base`, so memory that
// is reused by a later call (of any shape or protocol) can never look fresh.
// Eager calls number their steps from 2^31 (up to the 32-bit LL flags'
// restart point); captured calls from zero on counters of their own, leaving
// every counter and flag they consumed at zero.  No flag either kind leaves
// in a FIFO slot can match a step number of the other.
constexpr uint64_t kEagerBase = 1ull << 31;

struct Resources {
  int device = 0;
  char* fifo[3] = {nullptr, nullptr, nullptr};
  uint64_t fifo_conns[3] = {0, 0, 0};
  uint64_t* counters = nullptr;
  uint64_t* cap_counters = nullptr;   // captured calls' own counters, kept at zero between calls
  // A captured graph holds the addresses of the FIFO and counters it was
  // captured with.  Once the stream has captured a call, buffers replaced by
  // a larger allocation are kept here, alive for those graphs, until
  // ringar_release.
  bool captured_ever = false;
  std::vector<std::pair<void*, uint64_t>> retired;   // (address, bytes)
  uint64_t counter_conns = 0;
  // Two error words: [0] for eager calls, (call id << 8) | code, call ids
  // growing; [1] for captured calls, whose replays all carry the call id of
  // their capture and so need a word of their own.
  uint64_t* error = nullptr;
  uint64_t base = 0;
  uint64_t call_id = 0;
  uint64_t reported_call = 0;
  int wall_khz = 100000;
  int num_cus = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Resources> g_res;
std::map<long long, int> g_occupancy;   // (kernel, block) -> blocks per CU

// FIFO slots (unless `counters_only`) and counters for `conns` connections.
ringar_result_t ensure_conns(Resources& R, hipStream_t st, int proto, uint64_t conns, bool counters_only) {
  auto drop = [&R](void* p, uint64_t bytes) -> ringar_result_t {
    if (!p) return RINGAR_SUCCESS;
    if (R.captured_ever)
      R.retired.emplace_back(p, bytes);
    else
      HIP_TRY(hipFree(p));
    return RINGAR_SUCCESS;
  };
  ringar_result_t r;
  if (!counters_only && R.fifo_conns[proto] < conns) {
    HIP_TRY(hipStreamSynchronize(st));
    if ((r = drop(R.fifo[proto], R.fifo_conns[proto] * fifo_conn_bytes(proto))) != RINGAR_SUCCESS) return r;
    R.fifo[proto] = nullptr;
    R.fifo_conns[proto] = 0;
    const uint64_t bytes = conns * fifo_conn_bytes(proto);
    HIP_TRY(hipMalloc((void**)&R.fifo[proto], bytes));
    HIP_TRY(launch_fill((uint64_t*)R.fifo[proto], bytes / 8, 0, st));
    R.fifo_conns[proto] = conns;
  }
  if (R.counter_conns < conns) {
    HIP_TRY(hipStreamSynchronize(st));
    if ((r = drop(R.counters, R.counter_conns * kCounterWords * 8)) != RINGAR_SUCCESS) return r;
    if ((r = drop(R.cap_counters, R.counter_conns * kCounterWords * 8)) != RINGAR_SUCCESS) return r;
    R.counters = R.cap_counters = nullptr;
    R.counter_conns = 0;
    HIP_TRY(hipMalloc((void**)&R.counters, conns * kCounterWords * 8));
    HIP_TRY(launch_fill(R.counters, conns * kCounterWords, 0, st));
    HIP_TRY(hipMalloc((void**)&R.cap_counters, conns * kCounterWords * 8));
    HIP_TRY(launch_fill(R.cap_counters, conns * kCounterWords, 0, st));
    R.counter_conns = conns;
  }
  return RINGAR_SUCCESS;
}

ringar_result_t get_resources(hipStream_t st, Resources** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto key = std::make_pair(dev, st);
  auto it = g_res.find(key);
  if (it == g_res.end()) {
    Resources R;
    R.device = dev;
    HIP_TRY(hipDeviceGetAttribute(&R.wall_khz, hipDeviceAttributeWallClockRate, dev));
    HIP_TRY(hipDeviceGetAttribute(&R.num_cus, hipDeviceAttributeMultiprocessorCount, dev));
    HIP_TRY(hipMalloc((void**)&R.error, 16));
    HIP_TRY(launch_fill(R.error, 2, 0, st));
    R.base = kEagerBase;
    // Test hook: RINGAR_STEP_BASE, read when a stream's resources are
    // created, starts its step numbers there (e.g. just below the point
    // where the 32-bit LL flags are restarted).
    if (const char* v = getenv("RINGAR_STEP_BASE")) R.base = strtoull(v, nullptr, 0);
    it = g_res.emplace(key, R).first;
  }
  *out = &it->second;
  return RINGAR_SUCCESS;
}

// Restart the eager step numbers at kEagerBase: clear every flag and counter
// first.
ringar_result_t reset_steps(Resources& R, hipStream_t st) {
  for (int p = 0; p < 3; p++)
    if (R.fifo[p]) HIP_TRY(launch_fill((uint64_t*)R.fifo[p], R.fifo_conns[p] * fifo_conn_bytes(p) / 8, 0, st));
  if (R.counters) HIP_TRY(launch_fill(R.counters, R.counter_conns * kCounterWords, 0, st));
  R.base = kEagerBase;
  return RINGAR_SUCCESS;
}

// Resident wavefronts of the (dtype, op, proto) kernel on the current device,
// or 0 when no device is visible.  Cached per device and kernel.
uint64_t capacity_waves(int coll, int dtype, int op, int proto, bool cap) {
  static const int ndev = [] {
    int c = 0;
    if (hipGetDeviceCount(&c) != hipSuccess) {
      (void)hipGetLastError();
      c = 0;
    }
    return c;
  }();
  if (ndev == 0) return 0;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const long long key = (((((long long)dev * 4 + coll) * 8 + dtype) * 5 + op) * 4 + proto) * 2 + (cap ? 1 : 0);
  // the general form: the small one needs no more registers
  static std::mutex mu;
  static std::map<long long, uint64_t> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      max_active_blocks(coll, dtype, op, proto, false, cap, 256, &per_cu) != hipSuccess)
    return 0;
  uint64_t w = (uint64_t)cus * (uint64_t)per_cu * 4;   // 4 wavefronts per 256-thread block
  cache.emplace(key, w);
  return w;
}

bool overlaps(uintptr_t a, uintptr_t b, size_t len) { return a < b + len && b < a + len; }

// Buffers of rank r: send [sb[r], + slen), receive [rb[r], + rlen), both
// aligned to the element size.  Receive buffers must not overlap each other
// or any send buffer, except that a rank's buffers may share its own block
// in the collective's in-place form: receive == send for the AllReduce,
// receive == send + r * rlen for ReduceScatter, send == receive + r * slen
// for AllGather.  Send buffers may overlap each other (they are only read).
ringar_result_t check_buffers(int coll, void* const* sb, void* const* rb, size_t count, size_t es, int n) {
  if (!sb || !rb) return RINGAR_ERR_INVALID_ARGUMENT;
  for (int r = 0; r < n; r++) {
    if (!sb[r] || !rb[r]) return RINGAR_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)sb[r] % es) || ((uintptr_t)rb[r] % es)) return RINGAR_ERR_INVALID_ARGUMENT;
  }
  const size_t len = count * es;
  const size_t slen = coll == kReduceScatter ? (size_t)n * len : len;
  const size_t rlen = coll == kAllGather ? (size_t)n * len : len;
  for (int r = 0; r < n; r++) {
    const uintptr_t rr = (uintptr_t)rb[r];
    for (int q = 0; q < n; q++) {
      const uintptr_t rq = (uintptr_t)rb[q], sq = (uintptr_t)sb[q];
      if (q != r && rr < rq + rlen && rq < rr + rlen) return RINGAR_ERR_INVALID_USAGE;
      if (!(rr < sq + slen && sq < rr + rlen)) continue;
      bool in_place = false;
      if (q == r) {
        if (coll == kAllReduce) in_place = rr == sq;
        else if (coll == kReduceScatter) in_place = rr == sq + (uintptr_t)r * len;
        else in_place = sq == rr + (uintptr_t)r * len;
      }
      if (!in_place) return RINGAR_ERR_INVALID_USAGE;
    }
  }
  return RINGAR_SUCCESS;
}

ringar_result_t check_ring(const int* ring, int n) {
  if (!ring) return RINGAR_SUCCESS;
  // Follow the ring from index 0: it must visit every rank once and close
  // ([BOOK] §4, ncclBuildRings' check that a ring loops back and holds all
  // ranks).
  std::vector<char> seen(n, 0);
  for (int i = 0; i < n; i++) {
    int r = ring[i];
    if (r < 0 || r >= n || seen[r]) return RINGAR_ERR_INVALID_ARGUMENT;
    seen[r] = 1;
  }
  return RINGAR_SUCCESS;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char* ringar_result_string(ringar_result_t r) {
  switch (r) {
    case RINGAR_SUCCESS: return "success";
    case RINGAR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RINGAR_ERR_INVALID_USAGE: return "invalid usage";
    case RINGAR_ERR_INTERNAL: return "internal error";
    case RINGAR_ERR_DEVICE: return "device error";
    case RINGAR_ERR_ABORTED: return "aborted";
    case RINGAR_ERR_TIMEOUT: return "timeout";
  }
  return "unknown result";
}

const char* ringar_last_error(void) { return t_last_error.c_str(); }

ringar_result_t ringar_default_model(ringar_model_t* out) {
  if (!out) return RINGAR_ERR_INVALID_ARGUMENT;
  *out = default_model();
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_select(size_t bytes, int nranks, int nchannels, const ringar_model_t* model,
                              ringar_proto_t* out, double* predicted_us) {
  if (!out || nranks < 1 || nranks > kMaxRanks || nchannels < 0 || nchannels > kMaxChannels)
    return RINGAR_ERR_INVALID_ARGUMENT;
  ringar_model_t dm = default_model();
  const ringar_model_t& m = model ? *model : dm;
  if (nranks == 1) {
    *out = RINGAR_PROTO_SIMPLE;
    if (predicted_us) predicted_us[0] = predicted_us[1] = predicted_us[2] = 0.0;
    return RINGAR_SUCCESS;
  }
  int nch = nchannels > 0 ? nchannels : model_max_channels(m, nranks);
  double t[3];
  int p = select_proto(m, nranks, nch, bytes, env().proto_mask, t);
  if (p < 0) return RINGAR_ERR_INVALID_USAGE;
  *out = (ringar_proto_t)p;
  if (predicted_us) memcpy(predicted_us, t, sizeof(t));
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_tree(int nranks, int tree, int rank, int* parent, int* child0, int* child1) {
  if (nranks < 1 || nranks > kMaxRanks || tree < 0 || tree > 1 || rank < 0 || rank >= nranks || !parent ||
      !child0 || !child1)
    return RINGAR_ERR_INVALID_ARGUMENT;
  tree_links(nranks, tree, rank, parent, child0, child1);
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_select_algo(size_t bytes, int nranks, int nchannels, const ringar_model_t* model,
                                   ringar_algo_t* algo, ringar_proto_t* proto, double* predicted_us) {
  if (!algo || !proto || nranks < 1 || nranks > kMaxRanks || nchannels < 0 || nchannels > kMaxChannels)
    return RINGAR_ERR_INVALID_ARGUMENT;
  ringar_model_t dm = default_model();
  const ringar_model_t& m = model ? *model : dm;
  if (nranks == 1) {
    *algo = RINGAR_ALGO_RING;
    *proto = RINGAR_PROTO_SIMPLE;
    if (predicted_us)
      for (int i = 0; i < 6; i++) predicted_us[i] = 0.0;
    return RINGAR_SUCCESS;
  }
  const int nch = nchannels > 0 ? nchannels : model_max_channels(m, nranks);
  int a = 0, p = 0;
  if (!select_algo_proto(m, nranks, nch, bytes, env().algo_mask, env().proto_mask, &a, &p, predicted_us))
    return RINGAR_ERR_INVALID_USAGE;
  *algo = (ringar_algo_t)a;
  *proto = (ringar_proto_t)p;
  return RINGAR_SUCCESS;
}

// The (count, dtype) a collective's kernels work on: AllGather is a byte copy.
static void kernel_shape(int coll, size_t count, int dtype, size_t* kcount, int* kdtype) {
  const size_t es = elem_size(dtype);
  *kcount = coll == kAllGather ? count * es : count;
  *kdtype = coll == kAllGather ? (int)RINGAR_INT8 : dtype;
}

// The plan a launch uses: first without, then with the kernel's residency
// (`captured`: that of the captured form, whose line-protocol kernels hold
// fewer wavefronts; a lower residency only ever takes fewer lanes).
static ringar_result_t plan_for_launch(int coll, size_t count, int dtype, int op, int nranks, int nchannels,
                                int proto, const ringar_config_t* cfg, Plan* P, bool captured = false) {
  ringar_result_t r = make_plan(coll, count, dtype, nranks, nchannels, proto, cfg, 0, P, captured);
  if (r != RINGAR_SUCCESS) return r;
  if (count > 0 && nranks > 1) {
    const uint64_t cap =
        capacity_waves(P->kind, dtype, op, P->tree_split ? kSimpleSplitTree : P->proto, captured);
    if (cap && (r = make_plan(coll, count, dtype, nranks, nchannels, proto, cfg, cap, P, captured)) !=
                   RINGAR_SUCCESS)
      return r;
  }
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_plan_coll(ringar_coll_t coll, size_t count, ringar_dtype_t dtype, int nranks,
                                 int nchannels, ringar_proto_t proto, const ringar_config_t* cfg,
                                 ringar_plan_t* out) {
  if (!out || coll < RINGAR_ALLREDUCE || coll > RINGAR_ALL_GATHER) return RINGAR_ERR_INVALID_ARGUMENT;
  if (!elem_size(dtype)) return RINGAR_ERR_INVALID_ARGUMENT;
  size_t kcount;
  int kdtype;
  kernel_shape(coll, count, dtype, &kcount, &kdtype);
  Plan P;
  ringar_result_t r = plan_for_launch(coll, kcount, kdtype, 0, nranks, nchannels, proto, cfg, &P);
  if (r != RINGAR_SUCCESS) return r;
  const size_t es = elem_size(kdtype);
  out->proto = (ringar_proto_t)P.proto;
  out->nchannels = P.nch;
  out->chunk_bytes = P.chunk_bytes;
  out->chunk_elems = P.chunk_elems;
  out->align_elems = 16 / es;
  out->channel_elems = P.per_channel;
  out->lanes = P.lanes;
  out->fifo_depth = P.depth;
  out->small_slices = P.small ? 1 : 0;
  out->workgroups = P.grid;
  out->threads_per_group = P.block;
  out->max_steps = P.max_steps;
  for (int p = 0; p < 3; p++) {
    out->predicted_us[p] = P.times[p];
    out->predicted_tree_us[p] = P.tree_times[p];
    out->predicted_ring_us[p] = P.ring_times[p];
  }
  out->algo = P.kind == kTreeAllReduce ? RINGAR_ALGO_TREE : RINGAR_ALGO_RING;
  out->direct = P.direct ? 1 : 0;
  out->xcd_major = P.xcd_major ? 1 : 0;
  out->tree_split = P.tree_split ? 1 : 0;
  out->tree_waves_per_lane = P.tree_split ? P.tree_waves : 0;
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_plan(size_t count, ringar_dtype_t dtype, int nranks, int nchannels,
                            ringar_proto_t proto, const ringar_config_t* cfg, ringar_plan_t* out) {
  return ringar_plan_coll(RINGAR_ALLREDUCE, count, dtype, nranks, nchannels, proto, cfg, out);
}

ringar_result_t ringar_chunk_range(size_t count, ringar_dtype_t dtype, int nranks, int nchannels,
                                   size_t chunk_elems, int c, size_t loop_off, int k, size_t* lo,
                                   size_t* hi, size_t* klo, size_t* khi) {
  const size_t es = elem_size(dtype);
  if (!es || nranks < 1 || nchannels < 1 || c < 0 || c >= nchannels || k < 0 || k >= nranks ||
      chunk_elems == 0 || chunk_elems % (16 / es) || !lo || !hi || !klo || !khi)
    return RINGAR_ERR_INVALID_ARGUMENT;
  uint64_t per = channel_len(count, nchannels, (uint32_t)es), l, h;
  channel_bounds(count, per, c, &l, &h);
  *lo = l;
  *hi = h;
  const uint64_t len = h - l;
  if (loop_off >= len) {
    *klo = *khi = h;
    return RINGAR_SUCCESS;
  }
  uint64_t cur = loop_chunk(len, loop_off, nranks, chunk_elems, (uint32_t)es), s, n;
  chunk_bounds(len - loop_off, cur, k, &s, &n);
  *klo = l + loop_off + s;
  *khi = *klo + n;
  return RINGAR_SUCCESS;
}

// ---------------------------------------------------------------- scratch
// Memory of ringar_allreduce_noalloc, for callers that cannot allocate: FIFO
// slots, counters and an error word in one file-scope device array of fixed
// size, so that the entry point itself allocates nothing.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the array's name is only a stand-in: its device address on each device is
// taken once with hipGetSymbolAddress and kept in NoAllocState::base_ptr,
// which is what kernels and fills receive.
constexpr uint64_t kNoAllocFifoBytes = 64ull << 20;                  // FIFO slots
constexpr uint64_t kNoAllocCounterConns = 4096;                      // counter lines
constexpr uint64_t kNoAllocCounterBytes = kNoAllocCounterConns * kCounterWords * 8;
constexpr uint64_t kNoAllocBytes = kNoAllocFifoBytes + kNoAllocCounterBytes + 256;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
struct NoAllocState {
  bool ready = false;
  unsigned char* base_ptr = nullptr;   // device address of `scratch` on this device
  char* fifo = nullptr;                // [0, kNoAllocFifoBytes)
  uint64_t* counters = nullptr;        // kNoAllocCounterConns connections
  uint64_t* error = nullptr;           // (call id << 8) | code of the first failure
  uint64_t base = 0;                   // step base of the next call
  uint64_t call_id = 0;
  uint64_t reported_call = 0;
  int last_proto = -1;                 // protocol whose data the FIFO bytes hold
  uint64_t dirty_bytes = 0;            // FIFO bytes calls have written since the last clear
  int wall_khz = 100000;
  int num_cus = 0;
};
NoAllocState g_noalloc[kMaxDevices];   // guarded by g_mu

// Set-up on the first call on a device (that device current): the scratch
// array's device address, checked, then one clear of all of it.
ringar_result_t noalloc_state(hipStream_t st, NoAllocState** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return RINGAR_ERR_INVALID_USAGE;
  NoAllocState& S = g_noalloc[dev];
  if (!S.ready) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr || (uintptr_t)ptr % 256) {
      t_last_error = "hipGetSymbolAddress returned no usable address for the scratch array";
      return RINGAR_ERR_INTERNAL;
    }
    S.base_ptr = (unsigned char*)ptr;
    S.fifo = (char*)S.base_ptr;
    S.counters = (uint64_t*)(S.base_ptr + kNoAllocFifoBytes);
    S.error = (uint64_t*)(S.base_ptr + kNoAllocFifoBytes + kNoAllocCounterBytes);
    HIP_TRY(hipDeviceGetAttribute(&S.wall_khz, hipDeviceAttributeWallClockRate, dev));
    HIP_TRY(hipDeviceGetAttribute(&S.num_cus, hipDeviceAttributeMultiprocessorCount, dev));
    HIP_TRY(launch_fill((uint64_t*)S.base_ptr, kNoAllocBytes / 8, 0, st));
    S.base = kEagerBase;
    S.ready = true;
  }
  *out = &S;
  return RINGAR_SUCCESS;
}

// Scratch bytes a plan needs: FIFO slots of every connection (none for the
// direct form) and their counters.
bool noalloc_fits(const Plan& P, bool direct) {
  const uint64_t fifo = direct ? 0 : P.conns * fifo_conn_bytes(P.proto);
  return fifo <= kNoAllocFifoBytes && P.conns <= kNoAllocCounterConns;
}

// One ring collective.  count: elements per rank for the AllReduce, per
// block for ReduceScatter (recvcount) and AllGather (sendcount).
// noalloc: run on the device's scratch array instead of the stream's
// allocated resources; the plan keeps every choice that decides results
// (protocol, channels, chunk, algorithm) and takes fewer lanes when the
// scratch cannot hold the connections of the usual lane count.
static ringar_result_t run_collective(int coll, void* const* sendbuffs, void* const* recvbuffs, size_t count,
                               int udtype, int op, int nranks, int nchannels, int proto,
                               ringar_stream_t stream, const ringar_config_t* cfg, bool noalloc = false) {
  const size_t ues = elem_size(udtype);
  if (!ues || op < RINGAR_SUM || op > RINGAR_AVG) return RINGAR_ERR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > kMaxRanks) return RINGAR_ERR_INVALID_ARGUMENT;
  size_t kcount;
  int dtype;
  kernel_shape(coll, count, udtype, &kcount, &dtype);
  const size_t es = elem_size(dtype);
  Plan P;
  ringar_result_t r = plan_for_launch(coll, kcount, dtype, op, nranks, nchannels, proto, cfg, &P);
  if (r != RINGAR_SUCCESS) return r;
  if (cfg && (r = check_ring(cfg->ring_order, nranks)) != RINGAR_SUCCESS) return r;
  if (count == 0) return RINGAR_SUCCESS;                      // no-op, nothing enqueued
  if ((r = check_buffers(coll, sendbuffs, recvbuffs, count, ues, nranks)) != RINGAR_SUCCESS) return r;
  hipStream_t st = (hipStream_t)stream;
  if (nranks == 1) {                                          // one rank: a local copy
    if (sendbuffs[0] != recvbuffs[0])
      HIP_TRY(hipMemcpyAsync(recvbuffs[0], sendbuffs[0], count * ues, hipMemcpyDeviceToDevice, st));
    return RINGAR_SUCCESS;
  }
  count = kcount;
  // Under stream capture (a graph replays the call any number of times)
  // every collective runs its captured form: steps from zero on the
  // captured counters, every consumed flag and counter left at zero, nothing
  // allocated or cleared during capture.  The stream's resources must hold
  // the call's connections already (an eager call of the same shape on the
  // stream allocates them); the direct form is refused.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(st, &capture));
  const bool captured = capture != hipStreamCaptureStatusNone;
  if (captured && noalloc) {
    t_last_error = "the allocation-free entry point has no captured form";
    return RINGAR_ERR_INVALID_USAGE;
  }
  if (captured && (r = plan_for_launch(coll, kcount, dtype, op, nranks, nchannels, proto, cfg, &P, true)) !=
                      RINGAR_SUCCESS)
    return r;
  // Connections an eager call allocates on the stream: its own, and in the
  // split tree form also those of the captured (unsplit) form of the same
  // call, which takes other lanes, so that the stream can capture it next.
  uint64_t hold_conns = P.conns;
  if (!captured && !noalloc && P.tree_split) {
    Plan Q;
    if (plan_for_launch(coll, kcount, dtype, op, nranks, nchannels, proto, cfg, &Q, true) == RINGAR_SUCCESS)
      hold_conns = std::max(hold_conns, Q.conns);
  }

  // the direct form needs every rank out of place
  bool direct = P.direct;
  for (int q = 0; q < nranks && direct; q++)
    if (sendbuffs[q] == recvbuffs[q]) direct = false;
  if (captured && direct && P.direct_auto) direct = false;   // the library's choice: keep the FIFOs
  if (captured && direct) {
    t_last_error = "the direct form has no captured form";
    return RINGAR_ERR_INVALID_USAGE;
  }
  if (noalloc && !noalloc_fits(P, direct)) {
    // lanes change no result: take the most (a power of two below the
    // plan's) whose connections the scratch holds, unless they were forced
    const bool forced = (cfg && cfg->lanes) || env().lanes;
    bool found = false;
    if (!forced) {
      ringar_config_t c2;
      if (cfg) c2 = *cfg;
      else {
        memset(&c2, 0, sizeof(c2));
        c2.skip_rank = -1;
      }
      int L = 1;
      while (L * 2 < P.lanes) L *= 2;
      for (; L >= 1 && !found; L /= 2) {
        c2.lanes = L;
        Plan Q;
        if (plan_for_launch(coll, kcount, dtype, op, nranks, nchannels, proto, &c2, &Q) == RINGAR_SUCCESS &&
            noalloc_fits(Q, direct)) {
          P = Q;
          found = true;
        }
      }
    }
    if (!found) {
      char msg[256];
      snprintf(msg, sizeof(msg),
               "ringar_allreduce_noalloc: the call needs more than the %llu MiB of FIFO slots / %llu "
               "connections its scratch holds; use fewer channels or a smaller chunk",
               (unsigned long long)(kNoAllocFifoBytes >> 20), (unsigned long long)kNoAllocCounterConns);
      t_last_error = msg;
      return RINGAR_ERR_INVALID_USAGE;
    }
  }

  std::lock_guard<std::mutex> lock(g_mu);
  Resources* R = nullptr;
  NoAllocState* S = nullptr;
  if (noalloc) {
    if ((r = noalloc_state(st, &S)) != RINGAR_SUCCESS) return r;
  } else if (captured) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    auto it = g_res.find(std::make_pair(dev, st));
    if (it == g_res.end() || it->second.counter_conns < P.conns || it->second.fifo_conns[P.proto] < P.conns) {
      t_last_error = "under stream capture nothing is allocated: make one call of this shape on the stream first";
      return RINGAR_ERR_INVALID_USAGE;
    }
    R = &it->second;
  } else if ((r = get_resources(st, &R)) != RINGAR_SUCCESS) {
    return r;
  }
  const int num_cus = noalloc ? S->num_cus : R->num_cus;
  const int wall_khz = noalloc ? S->wall_khz : R->wall_khz;

  // All (rank, channel, lane) wavefronts wait on each other, so the whole
  // grid must be resident at once.
  // The vector path needs every user address 16-byte aligned, including the
  // block starts of the halves.
  int vec = (coll == kAllReduce || (count * es) % 16 == 0) ? 1 : 0;
  for (int q = 0; q < nranks; q++)
    if (((uintptr_t)sendbuffs[q] | (uintptr_t)recvbuffs[q]) % 16) vec = 0;
  const bool small = P.small && vec;
  // the kernel's selector: the protocol, or the split tree's own entry
  const int kproto = P.tree_split ? kSimpleSplitTree : P.proto;
  const long long okey = ((((long long)P.kind * 8 + dtype) * 5 + op) * 4 + kproto) * 4096 +
                         (captured ? 2048 : 0) + (small ? 1024 : 0) + P.block;
  auto oc = g_occupancy.find(okey);
  if (oc == g_occupancy.end()) {
    int per_cu = 0;
    HIP_TRY(max_active_blocks(P.kind, dtype, op, kproto, small, captured, P.block, &per_cu));
    oc = g_occupancy.emplace(okey, per_cu).first;
  }
  if ((long long)oc->second * num_cus < P.grid) return RINGAR_ERR_INVALID_USAGE;

  if (captured) R->captured_ever = true;
  if (noalloc) {
    // The FIFO bytes are shared by every protocol: data that another
    // protocol left in them could pass for a line flag, so they are cleared
    // whenever the protocol changes.  LL flags are 32-bit step numbers:
    // restart the numbering (clearing every flag and counter) before it wraps.
    const uint64_t touched = direct ? 0 : P.conns * fifo_conn_bytes(P.proto);
    if (!direct && P.proto != S->last_proto) {
      if (S->dirty_bytes) HIP_TRY(launch_fill((uint64_t*)S->fifo, S->dirty_bytes / 8, 0, st));
      S->dirty_bytes = 0;
      S->last_proto = P.proto;
    }
    S->dirty_bytes = std::max(S->dirty_bytes, touched);
    if (S->base + P.max_steps + 1 >= 0xFFFFFFF0ull) {
      HIP_TRY(launch_fill((uint64_t*)S->base_ptr, (kNoAllocFifoBytes + kNoAllocCounterBytes) / 8, 0, st));
      S->base = kEagerBase;
    }
  } else if (!captured) {
    // (the library's own direct choice still allocates the FIFOs, so that
    // the stream can capture the same call, which keeps them)
    if ((r = ensure_conns(*R, st, P.proto, hold_conns, direct && !P.direct_auto)) != RINGAR_SUCCESS) return r;
    // LL flags are 32-bit step numbers: restart the numbering before it wraps.
    if (R->base + P.max_steps + 1 >= 0xFFFFFFF0ull)
      if ((r = reset_steps(*R, st)) != RINGAR_SUCCESS) return r;
  }

  KernelArgs A;
  memset(&A, 0, sizeof(A));
  const int* ring = cfg ? cfg->ring_order : nullptr;
  for (int i = 0; i < nranks; i++) {
    int rank = ring ? ring[i] : i;
    A.send[i] = (const char*)sendbuffs[rank];
    A.recv[i] = (char*)recvbuffs[rank];
    A.rank_of[i] = rank;
  }
  A.count = count;
  A.per_channel = P.per_channel;
  A.chunk_elems = P.chunk_elems;
  if (noalloc) {
    A.base = S->base;
    A.counters = S->counters;
    A.error = S->error;
    A.call_id = ++S->call_id;
  } else {
    A.base = captured ? 0 : R->base;
    A.counters = captured ? R->cap_counters : R->counters;
    A.error = captured ? R->error + 1 : R->error;
    A.call_id = ++R->call_id;
  }
  A.abort_flag = cfg ? cfg->abort_flag : nullptr;
  uint32_t spin_ms = (cfg && cfg->spin_limit_ms) ? cfg->spin_limit_ms : env().spin_limit_ms;
  A.spin_ticks = (uint64_t)spin_ms * (uint64_t)wall_khz;
  A.nranks = nranks;
  A.nchannels = P.nch;
  A.lanes = P.lanes;
  A.depth = P.depth;
  A.lanes_per_block = P.lanes_per_block;
  A.xcd_major = P.xcd_major ? 1 : 0;
  A.skip_ring_index = -1;
  if (cfg && cfg->skip_rank >= 0 && cfg->skip_rank < nranks) {
    for (int i = 0; i < nranks; i++)
      if ((ring ? ring[i] : i) == cfg->skip_rank) A.skip_ring_index = i;
  }
  A.vec_ok = vec;
  A.direct = direct ? 1 : 0;
  A.fifo = direct ? nullptr : noalloc ? S->fifo : R->fifo[P.proto];

  if (P.kind == kTreeAllReduce) {
    // the tree runs over ranks 0..n-1 (a ring order does not apply)
    TreeArgs T;
    memset(&T, 0, sizeof(T));
    T.k = A;
    for (int i = 0; i < nranks; i++) {
      T.k.send[i] = (const char*)sendbuffs[i];
      T.k.recv[i] = (char*)recvbuffs[i];
      T.k.rank_of[i] = i;
    }
    T.k.skip_ring_index = (cfg && cfg->skip_rank >= 0 && cfg->skip_rank < nranks) ? cfg->skip_rank : -1;
    for (int t = 0; t < 2; t++)
      for (int v = 0; v < nranks; v++) {
        int u, c0, c1;
        tree_links(nranks, t, v, &u, &c0, &c1);
        T.parent[t][v] = (int8_t)u;
        T.child[t][0][v] = (int8_t)c0;
        T.child[t][1][v] = (int8_t)c1;
        if (u < 0) T.root[t] = v;
      }
    if (P.tree_split) {
      T.nroles = P.tree_waves;
      for (int t = 0; t < 2; t++) tree_split_roles(nranks, t, T.role_of[t]);
    }
    HIP_TRY(launch_tree(dtype, op, kproto, small, captured, T, P.grid, P.block, st));
  } else {
    HIP_TRY(launch_ring(coll, dtype, op, P.proto, small, captured, A, P.grid, P.block, st));
  }
  if (noalloc) S->base += P.max_steps + 1;
  else if (!captured) R->base += P.max_steps + 1;

  if (env().debug) {
    fprintf(stderr,
            "ringar: %s%s %zu bytes %s %s n=%d -> proto %s channels %d chunk %zu lanes %d "
            "depth %d%s%s grid %d x %d predicted LL %.1f LL128 %.1f Simple %.1f us\n",
            kCollName[P.kind], noalloc ? " (no alloc)" : "", count * es, kDtypeName[dtype], kOpName[op], nranks,
            kProtoName[P.proto], P.nch, P.chunk_bytes, P.lanes, P.depth, small ? " small" : "",
            direct ? " direct" : "", P.grid, P.block, P.times[0], P.times[1], P.times[2]);
  }
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_allreduce_ex(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                    ringar_dtype_t dtype, ringar_op_t op, int nranks,
                                    int nchannels, ringar_proto_t proto, ringar_stream_t stream,
                                    const ringar_config_t* cfg) {
  return run_collective(kAllReduce, sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto,
                        stream, cfg);
}

ringar_result_t ringar_allreduce_noalloc(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                         ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                         ringar_proto_t proto, ringar_stream_t stream,
                                         const ringar_config_t* cfg) {
  return run_collective(kAllReduce, sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto, stream,
                        cfg, true);
}

ringar_result_t ringar_reduce_scatter_ex(void* const* sendbuffs, void* const* recvbuffs, size_t recvcount,
                                         ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                         ringar_proto_t proto, ringar_stream_t stream,
                                         const ringar_config_t* cfg) {
  return run_collective(kReduceScatter, sendbuffs, recvbuffs, recvcount, dtype, op, nranks, nchannels,
                        proto, stream, cfg);
}

ringar_result_t ringar_reduce_scatter(void* const* sendbuffs, void* const* recvbuffs, size_t recvcount,
                                      ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                      ringar_proto_t proto, ringar_stream_t stream) {
  return ringar_reduce_scatter_ex(sendbuffs, recvbuffs, recvcount, dtype, op, nranks, nchannels, proto,
                                  stream, nullptr);
}

ringar_result_t ringar_all_gather_ex(void* const* sendbuffs, void* const* recvbuffs, size_t sendcount,
                                     ringar_dtype_t dtype, int nranks, int nchannels, ringar_proto_t proto,
                                     ringar_stream_t stream, const ringar_config_t* cfg) {
  return run_collective(kAllGather, sendbuffs, recvbuffs, sendcount, dtype, RINGAR_SUM, nranks, nchannels,
                        proto, stream, cfg);
}

ringar_result_t ringar_all_gather(void* const* sendbuffs, void* const* recvbuffs, size_t sendcount,
                                  ringar_dtype_t dtype, int nranks, int nchannels, ringar_proto_t proto,
                                  ringar_stream_t stream) {
  return ringar_all_gather_ex(sendbuffs, recvbuffs, sendcount, dtype, nranks, nchannels, proto, stream,
                              nullptr);
}

ringar_result_t ringar_allreduce(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                 ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                 ringar_proto_t proto, ringar_stream_t stream) {
  return ringar_allreduce_ex(sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto,
                             stream, nullptr);
}

ringar_result_t ringar_get_async_error(ringar_stream_t stream) {
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(st));
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto code_of = [](uint64_t w) {
    const int code = (int)(w & 0xff);
    if (code == RINGAR_ERR_ABORTED || code == RINGAR_ERR_TIMEOUT || code == RINGAR_ERR_INTERNAL)
      return (ringar_result_t)code;
    return RINGAR_ERR_INTERNAL;
  };
  auto it = g_res.find(std::make_pair(dev, st));
  if (it != g_res.end()) {
    Resources& R = it->second;
    uint64_t word[2] = {0, 0};
    HIP_TRY(hipMemcpy(word, R.error, 16, hipMemcpyDeviceToHost));
    const uint64_t call = word[0] >> 8;
    if (call > R.reported_call) {
      R.reported_call = call;
      return code_of(word[0]);
    }
    if (word[1] != 0) {
      // A captured call gave up: the wavefronts that stopped early left
      // counters and line flags behind that the next replay would take for
      // fresh ones.  Clear the word and everything the captured form counts
      // on being zero (its counters, the line-protocol FIFOs, and the
      // retired buffers older graphs may still use; eager calls never expect
      // zeros to be fresh, so clearing is safe for them too), so the graph
      // can be replayed again.
      if (R.cap_counters) HIP_TRY(launch_fill(R.cap_counters, R.counter_conns * kCounterWords, 0, st));
      for (int p = kLL; p <= kLL128; p++)
        if (R.fifo[p]) HIP_TRY(launch_fill((uint64_t*)R.fifo[p], R.fifo_conns[p] * fifo_conn_bytes(p) / 8, 0, st));
      for (auto& b : R.retired) HIP_TRY(launch_fill((uint64_t*)b.first, b.second / 8, 0, st));
      HIP_TRY(launch_fill(R.error + 1, 1, 0, st));
      HIP_TRY(hipStreamSynchronize(st));
      return code_of(word[1]);
    }
  }
  // the device's allocation-free calls (whatever stream they ran on)
  if (dev >= 0 && dev < kMaxDevices && g_noalloc[dev].ready) {
    NoAllocState& S = g_noalloc[dev];
    uint64_t word = 0;
    HIP_TRY(hipMemcpy(&word, S.error, 8, hipMemcpyDeviceToHost));
    const uint64_t call = word >> 8;
    if (call > S.reported_call) {
      S.reported_call = call;
      return code_of(word);
    }
  }
  return RINGAR_SUCCESS;
}

ringar_result_t ringar_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  HIP_TRY(hipGetDevice(&cur));
  for (auto& kv : g_res) {
    Resources& R = kv.second;
    HIP_TRY(hipSetDevice(R.device));
    HIP_TRY(hipDeviceSynchronize());
    for (int p = 0; p < 3; p++)
      if (R.fifo[p]) HIP_TRY(hipFree(R.fifo[p]));
    if (R.counters) HIP_TRY(hipFree(R.counters));
    if (R.cap_counters) HIP_TRY(hipFree(R.cap_counters));
    for (auto& p : R.retired) HIP_TRY(hipFree(p.first));
    if (R.error) HIP_TRY(hipFree(R.error));
  }
  g_res.clear();
  HIP_TRY(hipSetDevice(cur));
  return RINGAR_SUCCESS;
}

}  // extern "C"
