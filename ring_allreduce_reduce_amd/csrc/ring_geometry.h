// Geometry of one ring AllReduce launch: how the buffer is cut into channels,
// loops, chunks, lane parts and FIFO slices.  Used by the host (plan, step
// bounds) and by the kernel (addressing), so both agree by construction.
//
// Page rules ([BOOK] = "NCCL Source Code Deep Dive", [ARCH] = "NCCL
// architecture: topology, channels, algorithms and protocols"):
//   * channels own contiguous ranges of the buffer ([BOOK] §2.2); the length
//     per channel is rounded up to whole 16-byte units (the pages leave the
//     remainder open);
//   * a loop covers nranks chunks; the last partial loop uses chunks of
//     alignUp(ceil(rem / nranks), 16 B / elemSize) elements ([BOOK] §2.3);
//   * ring index i works on chunk (i + n - 1 - s) mod n at stage s ([BOOK] §2.3).
// MI355X additions (they change no result): each (rank, channel) chunk is
// split among `lanes` wavefronts in 1 KiB-aligned contiguous parts, each
// lane with its own FIFO; a lane's part is sent in FIFO slices of one slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define RA_HD __host__ __device__ __forceinline__

namespace ringar {

constexpr int kMaxRanks = 64;
constexpr int kMaxChannels = 64;
constexpr int kMaxLanes = 32;
// FIFO slots allocated per connection (the pages' NCCL_STEPS).  A call may
// cycle through fewer of them (its FIFO depth: 2, 4 or 8); a primitive may
// fill at most half the depth.
constexpr int kMaxSteps = 8;
constexpr int kMinSteps = 2;
constexpr int kMaxSlicesPerPart = kMaxSteps / 2;
constexpr uint32_t kLaneGranBytes = 1024; // lane parts start on 1 KiB boundaries
// LL128 lane parts: multiples of 8 lines of 120 data bytes, so that a part
// ends on a whole line (960 bytes, a multiple of 16 and of every element size)
constexpr uint32_t kLL128LaneGranBytes = 960;
constexpr uint32_t kSmallSliceBytes = 1024; // lane parts of the small-slice form (64 x 16 B)

// FIFO slot geometry per protocol.
constexpr uint32_t kSimpleSlotBytes = 32768;              // data bytes per slot
constexpr uint32_t kLLSlotLines = 2048;                    // 8-byte lines per slot (8 KiB of data)
constexpr uint32_t kLLSlotBytes = kLLSlotLines * 8;        // FIFO bytes per slot
constexpr uint32_t kLL128SlotLines = 256;                  // 128-byte lines per slot (30 KiB of data)
constexpr uint32_t kLL128SlotBytes = kLL128SlotLines * 128;// FIFO bytes per slot

// Groups the slices stream without per-lane conditions (a one-input
// primitive; two inputs take less): Simple, kUnroll 16-byte packets per
// lane of a 64-lane wavefront (the plan sizes Simple lane parts by it);
// LL128, kLL128WholeRows rows of 8 lines (one 16-byte packet per lane and
// row).
constexpr int kUnroll = 8;
constexpr uint32_t kSimpleGroupBytes = 64u * kUnroll * 16u;                 // 8 KiB
constexpr int kLL128WholeRows = 8;

enum Proto { kLL = 0, kLL128 = 1, kSimple = 2 };
// Launch kinds: the ring AllReduce and its halves (the public collective
// codes), and the tree AllReduce.
enum Coll { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2, kTreeAllReduce = 3 };
// Kernel selector for the split tree form (Simple), in place of the
// protocol when a tree kernel is looked up; never a protocol of a plan.
constexpr int kSimpleSplitTree = 3;

RA_HD uint64_t div_up(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
RA_HD uint64_t align_up(uint64_t a, uint64_t b) { return div_up(a, b) * b; }
RA_HD uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Elements of one 16-byte unit.
RA_HD uint64_t align_elems(uint32_t esize) { return 16 / esize; }

// Per-channel length before clipping to the buffer.
RA_HD uint64_t channel_len(uint64_t count, int nchannels, uint32_t esize) {
  return align_up(div_up(count, (uint64_t)nchannels), align_elems(esize));
}

// Channel c's element range [lo, hi).
RA_HD void channel_bounds(uint64_t count, uint64_t per_channel, int c, uint64_t* lo, uint64_t* hi) {
  *lo = min_u64(count, (uint64_t)c * per_channel);
  *hi = min_u64(count, *lo + per_channel);
}

// Chunk elements of the loop that starts `off` elements into a channel of
// `len` elements.
RA_HD uint64_t loop_chunk(uint64_t len, uint64_t off, int nranks, uint64_t chunk_elems,
                          uint32_t esize) {
  uint64_t loop = (uint64_t)nranks * chunk_elems;
  uint64_t rem = len - off;
  if (rem >= loop) return chunk_elems;
  return align_up(div_up(rem, (uint64_t)nranks), align_elems(esize));
}

// Chunk k of a loop with `rem` elements left and chunk size `cur`: start and
// length relative to the loop start (empty past the end).
RA_HD void chunk_bounds(uint64_t rem, uint64_t cur, int k, uint64_t* start, uint64_t* len) {
  uint64_t s = (uint64_t)k * cur;
  if (s >= rem) {
    *start = rem;
    *len = 0;
    return;
  }
  *start = s;
  *len = min_u64(cur, rem - s);
}

// Chunk visited by ring index i at stage s (0 <= s <= 2n-2).
RA_HD int stage_chunk(int i, int s, int nranks) { return (i - 1 - s + 2 * nranks) % nranks; }

// Lane part size of a loop whose chunks hold `cur` elements: the chunk size
// split over the lanes, rounded up to whole 1 KiB units.
RA_HD uint32_t lane_gran_bytes(int proto) { return proto == kLL128 ? kLL128LaneGranBytes : kLaneGranBytes; }
RA_HD uint64_t lane_part(uint64_t cur, int lanes, uint32_t esize, int proto) {
  return align_up(div_up(cur, (uint64_t)lanes), lane_gran_bytes(proto) / esize);
}

// Lane l's part of a chunk of `clen` elements (clen <= the loop's chunk
// size), given the loop's lane part size: [start, start + len).
RA_HD void lane_bounds(uint64_t clen, uint64_t part, int l, uint64_t* start, uint64_t* len) {
  uint64_t s = min_u64(clen, (uint64_t)l * part);
  *start = s;
  *len = min_u64(clen, s + part) - s;
}

// Elements one FIFO slot carries.
RA_HD uint64_t slot_elems(int proto, uint32_t esize) {
  if (proto == kSimple) return kSimpleSlotBytes / esize;
  if (proto == kLL) return (kLLSlotLines * 4) / esize;
  return (kLL128SlotLines * 120) / esize;
}

// LL lines of a slot: packet p (16 data bytes, 4 lines) keeps its word q in
// line (p / 64) * 256 + 64 q + p % 64, so that the 64 lanes of a wavefront,
// one packet each, load and store 64 consecutive lines (512 contiguous bytes)
// per instruction instead of every fourth line.
RA_HD uint32_t ll_line_index(uint32_t p, uint32_t q) { return (p >> 6) * 256u + q * 64u + (p & 63u); }
// Bytes of the slot prefix holding the lines of packets [0, npk).
RA_HD uint32_t ll_prefix_bytes(uint32_t npk) { return ((npk + 63u) / 64u) * 256u * 8u; }

// FIFO bytes of one slot and of one connection (kMaxSteps slots).
RA_HD uint64_t slot_bytes(int proto) {
  if (proto == kSimple) return kSimpleSlotBytes;
  if (proto == kLL) return kLLSlotBytes;
  return kLL128SlotBytes;
}
RA_HD uint64_t fifo_conn_bytes(int proto) { return (uint64_t)kMaxSteps * slot_bytes(proto); }

// Counters of one connection: tail and head, each on its own 128-byte line.
constexpr int kCounterWords = 32;   // uint64 words per connection (2 x 128 B)
constexpr int kTailWord = 0;
constexpr int kHeadWord = 16;
// A connection whose producer (consumer) runs as two half-lane wavefronts
// (the split tree below) has a second tail (head) word, one per half.
constexpr int kTail2Word = 8;
constexpr int kHead2Word = 24;

// MI355X dispatches the workgroups of a launch round-robin over its 8 XCDs
// (accelerator complex dies, each with its own L2): workgroup b runs on XCD
// b % 8.  A launch is `groups` groups of `members` workgroups (the ring
// indices of one channel and lane block, or the tree's roles).  The linear
// mapping puts member m of group g in workgroup g * members + m, so that
// neighbouring members sit on different XCDs.  The XCD-major mapping puts
// every member of group g on XCD g % 8: workgroup (g / 8 * members + m) * 8 +
// g % 8.  Its grid is 8 * members * ceil(groups / 8); the workgroups of a
// group number >= groups have no work.  Only speed depends on the mapping:
// every FIFO access is device-coherent.
constexpr int kXcds = 8;
RA_HD int launch_grid(int members, int groups, bool xcd_major) {
  return xcd_major ? kXcds * members * (int)div_up((uint64_t)groups, kXcds) : members * groups;
}
RA_HD void block_group(int b, int members, bool xcd_major, int* group, int* member) {
  if (!xcd_major) {
    *group = b / members;
    *member = b % members;
    return;
  }
  const int rest = b / kXcds;
  *member = rest % members;
  *group = (rest / members) * kXcds + b % kXcds;
}

// Connection feeding ring index i on channel c, lane l.
RA_HD uint64_t conn_index(int c, int i, int l, int nranks, int lanes) {
  return ((uint64_t)c * nranks + i) * lanes + l;
}

// Tree AllReduce connections: vertex v of channel c, lane l has an up
// connection (v -> its parent) and a down connection (its parent -> v).
enum TreeDir { kUp = 0, kDown = 1 };
RA_HD uint64_t tree_conn_index(int c, int v, int dir, int l, int nranks, int lanes) {
  return (((uint64_t)c * nranks + v) * 2 + dir) * lanes + l;
}

// Wavefront roles per (channel, lane) of the tree AllReduce: role v < n
// reduces vertex v into its parent (the root's role also starts the
// broadcast); role n + j broadcasts into the j-th vertex other than the root.
RA_HD int tree_roles(int nranks) { return 2 * nranks - 1; }

// Everything one launch needs, passed by value as kernel arguments.
struct KernelArgs {
  const char* send[kMaxRanks];   // by ring index
  char* recv[kMaxRanks];         // by ring index
  int rank_of[kMaxRanks];        // rank at ring index (blocks of the halves)
  uint64_t count;                // elements per rank (per block in the halves)
  uint64_t per_channel;
  uint64_t chunk_elems;
  uint64_t base;                 // step base of this call (absolute counters)
  char* fifo;                    // this protocol's FIFO region
  uint64_t* counters;            // kCounterWords per connection
  uint64_t* error;               // (call id << 8) | code of the first failure
  const volatile uint32_t* abort_flag;
  uint64_t spin_ticks;           // wall-clock ticks a wait may last
  uint64_t call_id;
  int nranks;
  int nchannels;
  int lanes;                     // wavefronts per (rank, channel)
  int depth;                     // FIFO slots in use per connection (2, 4, 8)
  int lanes_per_block;
  int skip_ring_index;           // -1: none
  int vec_ok;                    // all user pointers 16-byte aligned
  int direct;                    // Simple AllReduce writing the successor's receive buffer
  int xcd_major;                 // block ids map XCD-major (see block_group)
};

// Arguments of a tree AllReduce launch: the ring's, plus the two trees
// (channel c runs on tree c % 2), by rank: parent and children in child-slot
// order, -1 = none.
struct TreeArgs {
  KernelArgs k;
  int8_t parent[2][kMaxRanks];
  int8_t child[2][2][kMaxRanks];
  int root[2];
  // The split form (Simple): a role that moves four or more units of its
  // channel per element (the root's reduce role, the reduce and broadcast
  // roles of a vertex with two children) runs as two wavefronts, each on
  // half of every slice.  role_of[t][r] = vertex | broadcast << 6 |
  // half << 7 for the nroles wavefronts of a (channel, lane) on tree t.
  int nroles;
  uint8_t role_of[2][4 * kMaxRanks];
};

// Whether vertex v's reduce (broadcast) role splits in the split tree form:
// the root's reduce role, and either role of a vertex with two children.
RA_HD bool tree_role_splits(bool bcast, bool is_root, int nchildren) {
  return bcast ? nchildren == 2 : (is_root || nchildren == 2);
}

// The split form's handshake of one role (vertex v of tree t, its reduce or
// broadcast role): whether it splits, whether the producer of each of its
// inputs splits (then it waits for both tail words) and whether the consumer
// of each of its outputs splits (then it waits for both head words); inputs
// and outputs in the primitives' order, children in child-slot order.
struct SplitRole {
  bool my_split;
  bool in_split[2];
  bool out_split[2];
};
RA_HD int tree_children(const TreeArgs& ta, int t, int u) {
  return (ta.child[t][0][u] >= 0 ? 1 : 0) + (ta.child[t][1][u] >= 0 ? 1 : 0);
}
RA_HD SplitRole tree_split_role(const TreeArgs& ta, int t, int v, bool bcast) {
  const int root = ta.root[t];
  const int s0 = ta.child[t][0][v], s1 = ta.child[t][1][v];
  const int k0 = s0 >= 0 ? s0 : s1;
  const int k1 = s0 >= 0 ? s1 : -1;
  const int nk = (k0 >= 0 ? 1 : 0) + (k1 >= 0 ? 1 : 0);
  SplitRole r;
  r.my_split = tree_role_splits(bcast, v == root, nk);
  // the children's roles: their reduce roles send up, their broadcast roles
  // take the way down
  const bool up0 = k0 >= 0 && tree_role_splits(false, false, tree_children(ta, t, k0));
  const bool up1 = k1 >= 0 && tree_role_splits(false, false, tree_children(ta, t, k1));
  const bool down0 = k0 >= 0 && tree_role_splits(true, false, tree_children(ta, t, k0));
  const bool down1 = k1 >= 0 && tree_role_splits(true, false, tree_children(ta, t, k1));
  if (!bcast) {
    r.in_split[0] = up0;
    r.in_split[1] = up1;
    if (v == root) {
      r.out_split[0] = down0;
      r.out_split[1] = down1;
    } else {
      // the parent's reduce role reads the up connection
      const int p = ta.parent[t][v];
      r.out_split[0] = r.out_split[1] = tree_role_splits(false, p == root, tree_children(ta, t, p));
    }
  } else {
    // the down connection is written by the parent's broadcast role, or by
    // the root's reduce role
    const int p = ta.parent[t][v];
    r.in_split[0] = r.in_split[1] = tree_role_splits(p != root, p == root, tree_children(ta, t, p));
    r.out_split[0] = down0;
    r.out_split[1] = down1;
  }
  return r;
}

}  // namespace ringar
