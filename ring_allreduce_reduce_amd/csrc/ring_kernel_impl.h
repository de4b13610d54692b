// Ring AllReduce kernel for gfx950: n virtual ranks, all in one GPU.
//
// One launch runs every (ring index, channel, lane) as one wavefront.  Each
// wavefront walks the runRing primitive sequence of
// [ARCH] "NCCL architecture: topology, channels, algorithms and protocols",
// §九.4: send; (n-2) x recvReduceSend; recvReduceCopySend; (n-2) x
// recvCopySend; recv, once per loop of its channel.  A primitive moves the
// wavefront's part of one chunk through the FIFO to the successor ring index
// in slices of one FIFO slot, under one of the three protocols of §七.2:
//
//   Simple  data in the slot; the producer waits until its stores are
//           complete, then publishes the tail counter; the consumer polls the
//           tail, reads, then publishes the head counter that frees the slot.
//   LL      8-byte lines of 4 data bytes + 4 flag bytes, each written with a
//           single 64-bit store; the consumer re-reads a line until its flag
//           equals the step's flag.  No counter round trip for data.
//   LL128   128-byte lines of 120 data bytes + an 8-byte flag in bytes
//           120..127.  gfx950 does not promise that a 128-byte line written
//           by 8 lanes becomes visible at once (the pages rely on NVLink for
//           that), so the producer publishes a batch of line flags only after
//           its data stores have completed, and the consumer reads a line's
//           data only after it has seen that line's flag.
//
// FIFO accesses use device-coherent (sc1) loads and stores, which write
// through and read past the per-XCD L2 caches, so producer and consumer may
// sit on different XCDs.  Counters and flags are relaxed agent-scope atomics;
// ordering comes from waiting for the issuing wavefront's own outstanding
// memory operations (s_waitcnt vmcnt(0)) before a counter or flag is stored.
// Flags and counters hold absolute step numbers (call base + step + 1) that
// only grow across calls, so nothing is ever cleared between calls (§七.2:
// the LL flag is the step number, monotonic, never cleared by the receiver).
//
// Every wait is bounded: it gives up after spin_ticks of wall clock, when the
// host-mapped abort word is set, or when another wavefront of the same call
// has already given up; the first failure is recorded in the error word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_geometry.h"

namespace ringar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t s16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// ----------------------------------------------------------------- elements
// op(received a, local b); integers wrap, 16-bit floats go through fp32 and
// round to nearest-even, min/max keep the received value on ties.  OP codes:
// 0 sum, 1 prod, 2 min, 3 max, 4 avg (folds like sum; div() is its postOp:
// integers truncate toward zero, floats divide once in fp32 / fp64).
struct I8 {
  using T = uint8_t;
  __device__ static T div(T a, int n) { return (T)(int8_t)((int)(int8_t)a / n); }
  template <int OP> __host__ __device__ static T op(T a, T b) {
    if (OP == 0 || OP == 4) return (T)(a + b);
    if (OP == 1) return (T)((uint32_t)a * (uint32_t)b);
    int8_t sa = (int8_t)a, sb = (int8_t)b;
    if (OP == 2) return sb < sa ? b : a;
    return sb > sa ? b : a;
  }
  // The same op on the four bytes of a word at once: the sum with the carry
  // kept out of each byte's top bit; products and signed min / max on the
  // even and odd bytes as 16-bit lanes (packed 16-bit instructions), the
  // product's low byte and the sign-extended extremum packed back.  Fewer
  // instructions and registers than byte by byte, same results.
  template <int OP> __host__ __device__ static uint32_t op4(uint32_t a, uint32_t b) {
    if (OP == 0 || OP == 4) return ((a & 0x7f7f7f7fu) + (b & 0x7f7f7f7fu)) ^ ((a ^ b) & 0x80808080u);
    if (OP == 1) {
      const u16x2 pe = __builtin_bit_cast(u16x2, a & 0x00ff00ffu) * __builtin_bit_cast(u16x2, b & 0x00ff00ffu);
      const u16x2 po =
          __builtin_bit_cast(u16x2, (a >> 8) & 0x00ff00ffu) * __builtin_bit_cast(u16x2, (b >> 8) & 0x00ff00ffu);
      return (__builtin_bit_cast(uint32_t, pe) & 0x00ff00ffu) | ((__builtin_bit_cast(uint32_t, po) & 0x00ff00ffu) << 8);
    }
    const s16x2 ae = __builtin_bit_cast(s16x2, a << 8) >> 8, be = __builtin_bit_cast(s16x2, b << 8) >> 8;
    const s16x2 ao = __builtin_bit_cast(s16x2, a) >> 8, bo = __builtin_bit_cast(s16x2, b) >> 8;
    const s16x2 re = OP == 2 ? __builtin_elementwise_min(ae, be) : __builtin_elementwise_max(ae, be);
    const s16x2 ro = OP == 2 ? __builtin_elementwise_min(ao, bo) : __builtin_elementwise_max(ao, bo);
    return (__builtin_bit_cast(uint32_t, re) & 0x00ff00ffu) | ((__builtin_bit_cast(uint32_t, ro) & 0x00ff00ffu) << 8);
  }
};
struct I32 {
  using T = uint32_t;
  __device__ static T div(T a, int n) { return (T)((int32_t)a / n); }
  template <int OP> __device__ static T op(T a, T b) {
    if (OP == 0 || OP == 4) return a + b;
    if (OP == 1) return a * b;
    int32_t sa = (int32_t)a, sb = (int32_t)b;
    if (OP == 2) return sb < sa ? b : a;
    return sb > sa ? b : a;
  }
};
template <int OP> __device__ __forceinline__ float fop(float a, float b) {
  if (OP == 0 || OP == 4) return a + b;
  if (OP == 1) return a * b;
  if (OP == 2) return b < a ? b : a;
  return b > a ? b : a;
}
struct F16 {
  using T = uint16_t;
  __device__ static T div(T a, int n) {
    return __builtin_bit_cast(uint16_t, (_Float16)((float)__builtin_bit_cast(_Float16, a) / (float)n));
  }
  template <int OP> __device__ static T op(T a, T b) {
    float fa = (float)__builtin_bit_cast(_Float16, a);
    float fb = (float)__builtin_bit_cast(_Float16, b);
    return __builtin_bit_cast(uint16_t, (_Float16)fop<OP>(fa, fb));
  }
};
struct BF16 {
  using T = uint16_t;
  __device__ static float widen(T h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
  // round to nearest even: gfx950's conversion instruction (v_cvt_pk_bf16_f32)
  __device__ static T narrow(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
  template <int OP> __device__ static T op(T a, T b) { return narrow(fop<OP>(widen(a), widen(b))); }
  __device__ static T div(T a, int n) { return narrow(widen(a) / (float)n); }
};
struct F32 {
  using T = float;
  __device__ static T div(T a, int n) { return a / (float)n; }
  template <int OP> __device__ static T op(T a, T b) { return fop<OP>(a, b); }
};
struct F64 {
  using T = double;
  __device__ static T div(T a, int n) { return a / (double)n; }
  template <int OP> __device__ static T op(T a, T b) {
    if (OP == 0 || OP == 4) return a + b;
    if (OP == 1) return a * b;
    if (OP == 2) return b < a ? b : a;
    return b > a ? b : a;
  }
};

// Elementwise op over a 16-byte packet.
template <class E, int OP> __device__ __forceinline__ u32x4 vop(u32x4 a, u32x4 b) {
  if constexpr (std::is_same<E, I8>::value)
    return u32x4{I8::op4<OP>(a.x, b.x), I8::op4<OP>(a.y, b.y), I8::op4<OP>(a.z, b.z), I8::op4<OP>(a.w, b.w)};
  using T = typename E::T;
  constexpr int N = 16 / sizeof(T);
  struct P { T v[N]; };
  P pa = __builtin_bit_cast(P, a), pb = __builtin_bit_cast(P, b), pr;
#pragma unroll
  for (int e = 0; e < N; e++) pr.v[e] = E::template op<OP>(pa.v[e], pb.v[e]);
  return __builtin_bit_cast(u32x4, pr);
}

// Elementwise postOp division over a 16-byte packet.
template <class E> __device__ __forceinline__ u32x4 vdiv(u32x4 a, int n) {
  using T = typename E::T;
  constexpr int N = 16 / sizeof(T);
  struct P { T v[N]; };
  P pa = __builtin_bit_cast(P, a);
#pragma unroll
  for (int e = 0; e < N; e++) pa.v[e] = E::div(pa.v[e], n);
  return __builtin_bit_cast(u32x4, pa);
}

// ----------------------------------------------------------------- memory
constexpr int kSC1 = 16;   // device-coherent: write through / read past L2
constexpr int kNT = 2;     // streaming hint for user buffers
constexpr int kVolatile = (int)0x80000000u;   // re-read on every poll (compiler side)

// Buffer resource over [base, base + bytes).  Every caller passes values that
// are the same in all lanes of the wavefront; reading them from the first
// lane tells the compiler so, which keeps the resource in scalar registers
// (a resource it cannot prove uniform makes it loop over the distinct values
// around every buffer access).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

template <int AUX> __device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}
template <int AUX> __device__ __forceinline__ void st16(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, AUX);
}
template <int AUX> __device__ __forceinline__ u32x4 ld8(rsrc_t r, uint32_t off) {
  u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
  return u32x4{v.x, v.y, 0u, 0u};
}
template <int AUX> __device__ __forceinline__ void st8(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, (int)off, 0, AUX);
}

// Element-wise access to the first `nb` bytes (a multiple of the element
// size, < 16) of a packet at byte offset `off`: for ragged tails and for
// buffers that are not 16-byte aligned.
template <class E, int AUX> __device__ __forceinline__ u32x4 ld_part(rsrc_t r, uint32_t off, uint32_t nb) {
  using T = typename E::T;
  constexpr int N = 16 / sizeof(T);
  struct P { T v[N]; };
  P p;
#pragma unroll
  for (int e = 0; e < N; e++) {
    T x = 0;
    if ((uint32_t)(e * sizeof(T)) < nb) {
      uint32_t o = off + e * sizeof(T);
      if constexpr (sizeof(T) == 1) x = __builtin_amdgcn_raw_buffer_load_b8(r, (int)o, 0, AUX);
      else if constexpr (sizeof(T) == 2) x = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, AUX);
      else if constexpr (sizeof(T) == 4) x = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, (int)o, 0, AUX));
      else x = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, AUX));
    }
    p.v[e] = x;
  }
  return __builtin_bit_cast(u32x4, p);
}
template <class E, int AUX> __device__ __forceinline__ void st_part(u32x4 v, rsrc_t r, uint32_t off, uint32_t nb) {
  using T = typename E::T;
  constexpr int N = 16 / sizeof(T);
  struct P { T v[N]; };
  P p = __builtin_bit_cast(P, v);
#pragma unroll
  for (int e = 0; e < N; e++) {
    if ((uint32_t)(e * sizeof(T)) < nb) {
      uint32_t o = off + e * sizeof(T);
      if constexpr (sizeof(T) == 1) __builtin_amdgcn_raw_buffer_store_b8(p.v[e], r, (int)o, 0, AUX);
      else if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(p.v[e], r, (int)o, 0, AUX);
      else if constexpr (sizeof(T) == 4) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, p.v[e]), r, (int)o, 0, AUX);
      else __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, p.v[e]), r, (int)o, 0, AUX);
    }
  }
}

__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- waiting
enum { kErrInternal = 3, kErrAborted = 5, kErrTimeout = 6 };

__device__ __forceinline__ void record_error(const KernelArgs& a, int code) {
  __hip_atomic_fetch_max(a.error, (a.call_id << 8) | (uint64_t)code, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

struct Waiter {
  const KernelArgs* a;
  uint64_t t0;
  uint32_t spins;
  __device__ void start() { t0 = 0; spins = 0; }
  // One idle round of a wait loop; false when the wait must give up.
  __device__ __forceinline__ bool idle() {
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 127u) != 0) return true;
    uint64_t now = wall_clock64();
    if (t0 == 0) t0 = now;
    uint64_t err = ld_relaxed(a->error);
    if ((err >> 8) == a->call_id) return false;                 // a peer gave up
    int code = 0;
    if (a->abort_flag && __hip_atomic_load(a->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
      code = kErrAborted;
    else if (now - t0 > a->spin_ticks)
      code = kErrTimeout;
    if (code) {
      record_error(*a, code);
      return false;
    }
    return true;
  }
};

// The first lane's value of a 64-bit word, as a wavefront-uniform value.
// readfirstlane returns a signed int: each half is taken back as unsigned
// before it is widened, or a low half with bit 31 set would sign-extend into
// the high half (and a counter at or above 2^31 would look enormous).
__device__ __forceinline__ uint64_t first_lane_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Waits until *p >= v (wavefront-uniform).  `seen` is the largest value of
// *p this wavefront has observed; counters only grow, so a wait it already
// satisfies costs no memory round trip, and a poll records what it saw.
__device__ __forceinline__ bool wait_ge(Waiter& w, const uint64_t* p, uint64_t v, uint64_t& seen) {
  if (seen >= v) return true;
  w.start();
  while (true) {
    const uint64_t x = ld_relaxed(p);
    // every lane loads the same word; vote so the exit is uniform
    if (__all(x >= v)) {
      seen = first_lane_u64(x);
      break;
    }
    if (!w.idle()) return false;
  }
  compiler_fence();
  return true;
}

// ----------------------------------------------------------------- one lane
struct Conn {
  char* fifo;          // kMaxSteps slots, the first depth of them in use
  uint64_t* tail;      // written by the producer
  uint64_t* head;      // written by the consumer
};

template <int PROTO> __device__ __forceinline__ Conn conn_at(const KernelArgs& a, uint64_t idx) {
  return Conn{a.fifo + idx * fifo_conn_bytes(PROTO), a.counters + idx * kCounterWords + kTailWord,
              a.counters + idx * kCounterWords + kHeadWord};
}
// The second half's counter words of a connection (split tree form).
__device__ __forceinline__ uint64_t* tail2_of(const Conn& c) { return c.tail + (kTail2Word - kTailWord); }
__device__ __forceinline__ uint64_t* head2_of(const Conn& c) { return c.head + (kHead2Word - kHeadWord); }

// A wavefront's connections: one input and one output on the ring; a tree
// vertex receives from up to two children and sends to up to two.  All
// connections of a wavefront move in lockstep (one slice is one step on
// each), so they share the step numbers.
struct Lane {
  const KernelArgs* a;
  Conn in[2], out[2];
  const char* src;     // own send buffer
  char* dst;           // own receive buffer
  char* peer;          // the successor's receive buffer (direct form)
  uint64_t sstep, rstep;
  uint64_t tail_seen[2];  // largest tail of each input connection seen so far
  uint64_t head_seen[2];  // largest head of each output connection seen so far
  int lane;            // lane within the wavefront
  Waiter w;
  bool cap;            // a captured call (the kernel instance's constant)
  uint32_t zbytes;     // captured line protocols: most slot bytes a slice read
  // split tree form (primitives flagged kSplit): whether the producer of
  // each input / the consumer of each output runs as two halves, and
  // whether this wavefront is one half of its role (and which)
  bool in_split[2], out_split[2], my_split;
  int my_half;
  uint64_t tail2_seen[2], head2_seen[2];
#ifdef RINGAR_ROLE_PROFILE
  uint64_t w_in, w_out, n_sl;   // wall-clock ticks waiting for inputs / output slots, slices
#endif
};

#ifdef RINGAR_ROLE_PROFILE
// Role profile (a diagnostic build, never the library's own): per wavefront
// of a tree launch, its first and last wall-clock tick, the ticks its Simple
// slices waited for their inputs and for free output slots, the slices, and
// its role (vertex, broadcast bit, children, root bit; in the split form
// whether the role splits and which half this is).  Written by lane 0 of
// every wavefront of the eager Simple tree kernels of one element type's
// translation unit.
constexpr int kRoleProfileWaves = 4096;
static __device__ unsigned long long g_role_profile[kRoleProfileWaves][8];
#endif

// Primitive flags: receive (from input 0, and input 1 with kRecv2), send (to
// output 0, and output 1 with kSend2), read the own send buffer, write the
// own receive buffer.
enum : int { kRecv = 1, kSend = 2, kSrc = 4, kDst = 8, kRecv2 = 16, kSend2 = 32, kPost = 64, kSplit = 128 };
// kSplit: the split tree form; the Lane's split fields say which of the
// connection's counter words to wait for and write, and the slice is this
// wavefront's half (see slice_simple).
// kPost: the primitive where a chunk becomes final applies the op's postOp
// (the average's division by n, [ARCH] §九.4 recvReduceCopySend's postOp).
template <int OP> constexpr int post_flag() { return OP == 4 ? kPost : 0; }

// Frees the input slots just read: publishes head = base + step + 1.  Every
// load of a slot has returned its data (the values were consumed above),
// so the producer may overwrite it; the wavefront's own stores need not be
// complete, and waiting for them here would add a round trip to every step.
template <int F> __device__ __forceinline__ void release_slot(Lane& L) {
  compiler_fence();
  const bool second = (F & kSplit) && L.my_split && L.my_half;
  st_relaxed(second ? head2_of(L.in[0]) : L.in[0].head, L.a->base + L.rstep + 1);
  if (F & kRecv2) st_relaxed(second ? head2_of(L.in[1]) : L.in[1].head, L.a->base + L.rstep + 1);
  L.rstep++;
}

// Captured calls (a graph may replay one any number of times) run kernel
// instances of their own: their steps count from zero on counters of their
// own, and they leave every counter and flag they consumed at zero.  Within
// a call every flag is a distinct step number, so a slot's lines need to be
// clean only for the next replay: after its last step the receiver of a
// connection zeroes the slot bytes it read (the largest slice's prefix of
// every slot the call used) and the tail and head.  Its producer has
// written its last line, published its last tail and read its last head by
// then.  Eager calls count from 2^31 up, so no flag either kind leaves
// behind can match the other's.
template <int PROTO> __device__ __forceinline__ void finish_input(const Lane& L, const Conn& c) {
  if (PROTO != kSimple) {
    const uint32_t slot = PROTO == kLL ? kLLSlotBytes : kLL128SlotBytes;
    const uint64_t nslots = min_u64(L.rstep, (uint64_t)L.a->depth);
    for (uint64_t sl = 0; sl < nslots; sl++) {
      char* base = c.fifo + sl * slot;
      if (PROTO == kLL) {
        for (uint32_t off = (uint32_t)L.lane * 8u; off < L.zbytes; off += 64u * 8u)
          st_relaxed((uint64_t*)(base + off), 0);   // whole lines: data and flag
      } else {
        for (uint32_t line = (uint32_t)L.lane; line * 128u < L.zbytes; line += 64u)
          st_relaxed((uint64_t*)(base + (size_t)line * 128u + 120u), 0);   // the flag
      }
    }
  }
  st_relaxed(c.tail, 0);
  st_relaxed(c.head, 0);
}

// Waits for the tails of the inputs and for free slots on the outputs of
// the next step.
template <int F> __device__ __forceinline__ bool wait_inputs(Lane& L) {
  const KernelArgs& a = *L.a;
  const uint64_t need = a.base + L.rstep + 1;
  if ((F & kRecv) && !wait_ge(L.w, L.in[0].tail, need, L.tail_seen[0])) return false;
  if ((F & kRecv2) && !wait_ge(L.w, L.in[1].tail, need, L.tail_seen[1])) return false;
  if constexpr ((F & kSplit) != 0) {
    // a split producer publishes each half's tail on its own word
    if ((F & kRecv) && L.in_split[0] && !wait_ge(L.w, tail2_of(L.in[0]), need, L.tail2_seen[0])) return false;
    if ((F & kRecv2) && L.in_split[1] && !wait_ge(L.w, tail2_of(L.in[1]), need, L.tail2_seen[1])) return false;
  }
  return true;
}
template <int F> __device__ __forceinline__ bool wait_outputs(Lane& L) {
  const KernelArgs& a = *L.a;
  if (L.sstep < (uint64_t)a.depth) return true;
  const uint64_t need = a.base + L.sstep + 1 - a.depth;
  if ((F & kSend) && !wait_ge(L.w, L.out[0].head, need, L.head_seen[0])) return false;
  if ((F & kSend2) && !wait_ge(L.w, L.out[1].head, need, L.head_seen[1])) return false;
  if constexpr ((F & kSplit) != 0) {
    // a split consumer frees each half of a slot on its own word
    if ((F & kSend) && L.out_split[0] && !wait_ge(L.w, head2_of(L.out[0]), need, L.head2_seen[0])) return false;
    if ((F & kSend2) && L.out_split[1] && !wait_ge(L.w, head2_of(L.out[1]), need, L.head2_seen[1])) return false;
  }
  return true;
}

// Publishes the tails of the outputs after the step's data stores.
template <int F> __device__ __forceinline__ void publish_tails(Lane& L) {
  wait_mem();
  const bool second = (F & kSplit) && L.my_split && L.my_half;
  st_relaxed(second ? tail2_of(L.out[0]) : L.out[0].tail, L.a->base + L.sstep + 1);
  if (F & kSend2) st_relaxed(second ? tail2_of(L.out[1]) : L.out[1].tail, L.a->base + L.sstep + 1);
  L.sstep++;
}

// kUnroll (ring_geometry.h): 16-byte packets per lane in flight per source.
// Three sources (a tree vertex with two children) take 6 packets each (tree
// Simple, fp32 sum, n = 8, 64 MiB per rank, 32 channels on MI355X: 529 us
// with 4, 505 us with 6; the tree kernels keep their occupancy).
constexpr int kTwoInputUnroll = 6;

// Result of one packet: the local operand b folded with what was received
// from input 0 (a) and then input 1 (a2), each hop as op(received, local);
// or the received packet alone when there is no local operand.
template <class E, int OP, int F> __device__ __forceinline__ u32x4 combine(u32x4 a, u32x4 a2, u32x4 b, int n) {
  static_assert(!(F & kRecv2) || ((F & kRecv) && (F & kSrc)), "a second input is folded into a local operand");
  static_assert(!(F & kSend2) || (F & kSend), "a second output needs the first");
  static_assert(!(F & kPost) || ((F & kRecv) && (F & kSrc)), "the postOp follows the last fold");
  if constexpr ((F & kRecv) && (F & kSrc)) {
    u32x4 r = vop<E, OP>(a, b);
    if constexpr (F & kRecv2) r = vop<E, OP>(a2, r);
    if constexpr (F & kPost) r = vdiv<E>(r, n);
    return r;
  } else if constexpr (F & kRecv) {
    return a;
  } else {
    return b;
  }
}

// --- Simple: one slice = one slot ------------------------------------------
template <class E, int OP, int F>
__device__ __forceinline__ bool slice_simple(Lane& L, uint64_t es0, uint64_t ed0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
#ifdef RINGAR_ROLE_PROFILE
  const uint64_t t0 = wall_clock64();
  if (!wait_inputs<F>(L)) return false;
  const uint64_t t1 = wall_clock64();
  if (!wait_outputs<F>(L)) return false;
  L.w_in += t1 - t0;
  L.w_out += wall_clock64() - t1;
  L.n_sl++;
#else
  if (!wait_inputs<F>(L) || !wait_outputs<F>(L)) return false;
#endif
  uint32_t rslot = (uint32_t)(L.rstep & (a.depth - 1)) * kSimpleSlotBytes;
  uint32_t sslot = (uint32_t)(L.sstep & (a.depth - 1)) * kSimpleSlotBytes;
  uint32_t slot_bytes = kSimpleSlotBytes;
  if constexpr ((F & kSplit) != 0) {
    // one half of a split role: the first (second) half of the slice's
    // elements, cut at a whole 16-byte unit; in every slot it reads or
    // writes, the same half (the other wavefront of the role takes the
    // rest, and an unsplit peer the whole slot)
    if (L.my_split) {
      const uint32_t unit = 16 / (uint32_t)sizeof(typename E::T);
      const uint32_t hb = min((uint32_t)div_up(div_up(nelem, 2), unit) * unit, nelem);
      const uint32_t skip = L.my_half ? hb : 0;
      es0 += skip;
      ed0 += skip;
      nelem = L.my_half ? nelem - hb : hb;
      nbytes = nelem * (uint32_t)sizeof(typename E::T);
      rslot += skip * (uint32_t)sizeof(typename E::T);
      sslot += skip * (uint32_t)sizeof(typename E::T);
      slot_bytes -= skip * (uint32_t)sizeof(typename E::T);
    }
  }
  rsrc_t rin = make_rsrc(L.in[0].fifo + rslot, slot_bytes);
  rsrc_t rin2 = make_rsrc(L.in[(F & kRecv2) ? 1 : 0].fifo + rslot, slot_bytes);
  rsrc_t rout = make_rsrc(L.out[0].fifo + sslot, slot_bytes);
  rsrc_t rout2 = make_rsrc(L.out[(F & kSend2) ? 1 : 0].fifo + sslot, slot_bytes);
  rsrc_t rsrc_ = make_rsrc(L.src + es0 * sizeof(typename E::T), nbytes);
  rsrc_t rdst = make_rsrc(L.dst + ed0 * sizeof(typename E::T), nbytes);
  const uint32_t npk = (nbytes + 15) / 16;               // 16-byte packets
  const uint32_t nfull = a.vec_ok ? nbytes / 16 : 0;     // taken on the vector path
  // three sources in flight (a tree vertex with two children) take a
  // smaller unroll and the division of an average half, so that the kernel
  // keeps the ring's register budget (occupancy 4)
  constexpr int U = (F & kPost) ? kUnroll / 2 : (F & kRecv2) ? kTwoInputUnroll : kUnroll;
  // Whole groups of 64U packets: every lane in range, so the loads carry no
  // condition and all of a group's loads are issued before its first store.
  // (A per-lane condition turns each load into its own branch, and the
  // compiler then waits for every outstanding store at the top of each
  // group.)
  const uint32_t nmain = nfull - nfull % (64u * U);
  for (uint32_t p0 = 0; p0 < nmain; p0 += 64 * U) {
    u32x4 va[U], va2[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t off = (p0 + u * 64 + L.lane) * 16;
      if (F & kRecv) va[u] = ld16<kSC1>(rin, off);
      if (F & kRecv2) va2[u] = ld16<kSC1>(rin2, off);
      if (F & kSrc) vb[u] = ld16<kNT>(rsrc_, off);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t off = (p0 + u * 64 + L.lane) * 16;
      const u32x4 r = combine<E, OP, F>(va[u], va2[u], vb[u], a.nranks);
      if (F & kSend) st16<kSC1>(r, rout, off);
      if (F & kSend2) st16<kSC1>(r, rout2, off);
      if (F & kDst) st16<kNT>(r, rdst, off);
    }
  }
  // the last partial group: per-lane conditions
  for (uint32_t p0 = nmain; p0 < nfull; p0 += 64 * U) {
    u32x4 va[U], va2[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      const bool in = p < nfull;
      if (F & kRecv) va[u] = in ? ld16<kSC1>(rin, p * 16) : u32x4{0u, 0u, 0u, 0u};
      if (F & kRecv2) va2[u] = in ? ld16<kSC1>(rin2, p * 16) : u32x4{0u, 0u, 0u, 0u};
      if (F & kSrc) vb[u] = in ? ld16<kNT>(rsrc_, p * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      if (p >= nfull) continue;
      const u32x4 r = combine<E, OP, F>(va[u], va2[u], vb[u], a.nranks);
      if (F & kSend) st16<kSC1>(r, rout, p * 16);
      if (F & kSend2) st16<kSC1>(r, rout2, p * 16);
      if (F & kDst) st16<kNT>(r, rdst, p * 16);
    }
  }
  // The ragged last packet, or every packet when a user buffer is not
  // 16-byte aligned: element-wise on the user side.
#pragma unroll 1
  for (uint32_t p = nfull + L.lane; p < npk; p += 64) {
    const uint32_t off = p * 16, nb = min(16u, nbytes - off);
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, x2 = x, y = x;
    if (F & kRecv) x = ld16<kSC1>(rin, off);
    if (F & kRecv2) x2 = ld16<kSC1>(rin2, off);
    if (F & kSrc) y = ld_part<E, kNT>(rsrc_, off, nb);
    const u32x4 r = combine<E, OP, F>(x, x2, y, a.nranks);
    if (F & kSend) st16<kSC1>(r, rout, off);
    if (F & kSend2) st16<kSC1>(r, rout2, off);
    if (F & kDst) st_part<E, kNT>(r, rdst, off, nb);
  }
  if (F & kSend) publish_tails<F>(L);
  if (F & kRecv) release_slot<F>(L);
  return true;
}

// --- LL: 8-byte lines, 4 data bytes + 4 flag bytes ------------------------
__device__ __forceinline__ uint64_t ll_line(uint32_t data, uint32_t flag) {
  return ((uint64_t)flag << 32) | data;
}

__device__ __forceinline__ bool ll_ready(uint64_t line, uint32_t flag) {
  return (uint32_t)(line >> 32) == flag;
}

// Polls the 4 lines of packet p until all carry `flag`; wavefront-uniform
// over the active lanes.
__device__ __forceinline__ bool ll_recv4(Waiter& w, const uint64_t* lin, uint32_t p, bool active,
                                         uint32_t flag, uint64_t (&ln)[4]) {
#pragma unroll
  for (int q = 0; q < 4; q++) ln[q] = active ? ld_relaxed(lin + ll_line_index(p, q)) : ll_line(0, flag);
  w.start();
  while (true) {
    bool ok = ll_ready(ln[0], flag) && ll_ready(ln[1], flag) && ll_ready(ln[2], flag) &&
              ll_ready(ln[3], flag);
    if (__all(ok)) return true;
    if (!w.idle()) return false;
#pragma unroll
    for (int q = 0; q < 4; q++)
      if (!ll_ready(ln[q], flag)) ln[q] = ld_relaxed(lin + ll_line_index(p, q));
  }
}

// One LL line through a buffer resource (8-byte, device-coherent).
__device__ __forceinline__ uint64_t ll_load(rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kSC1 | kVolatile);
  return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ void ll_store(rsrc_t r, uint32_t off, uint32_t data, uint32_t flag) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{data, flag}, r, (int)off, 0, kSC1);
}

__device__ __forceinline__ void ll_send4(uint64_t* lout, uint32_t p, u32x4 r, uint32_t flag) {
  st_relaxed(lout + ll_line_index(p, 0), ll_line(r.x, flag));
  st_relaxed(lout + ll_line_index(p, 1), ll_line(r.y, flag));
  st_relaxed(lout + ll_line_index(p, 2), ll_line(r.z, flag));
  st_relaxed(lout + ll_line_index(p, 3), ll_line(r.w, flag));
}

template <class E, int OP, int F>
__device__ __forceinline__ bool slice_ll(Lane& L, uint64_t es0, uint64_t ed0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  const uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
  if (!wait_outputs<F>(L)) return false;
  constexpr int NI = (F & kRecv2) ? 2 : 1;   // inputs
  const uint32_t fin = (uint32_t)(a.base + L.rstep + 1);
  const uint32_t fout = (uint32_t)(a.base + L.sstep + 1);
  const uint64_t rslot = (L.rstep & (a.depth - 1)) * kLLSlotBytes;
  const uint64_t sslot = (L.sstep & (a.depth - 1)) * kLLSlotBytes;
  const uint64_t* lin[2] = {(const uint64_t*)(L.in[0].fifo + rslot),
                            (const uint64_t*)(L.in[NI - 1].fifo + rslot)};
  uint64_t* lout = (uint64_t*)(L.out[0].fifo + sslot);
  uint64_t* lout2 = (uint64_t*)(L.out[(F & kSend2) ? 1 : 0].fifo + sslot);
  rsrc_t rsrc_ = make_rsrc(L.src + es0 * sizeof(typename E::T), nbytes);
  rsrc_t rdst = make_rsrc(L.dst + ed0 * sizeof(typename E::T), nbytes);
  const uint32_t npk = (nbytes + 15) / 16;   // a packet = 16 data bytes = 4 lines
  const uint32_t nfull = a.vec_ok ? nbytes / 16 : 0;
  if ((F & kRecv) && L.cap) L.zbytes = max(L.zbytes, ll_prefix_bytes(npk));   // slot bytes read (see finish_input)
  constexpr int U = NI == 2 ? 2 : 4;   // packets per lane per poll (registers)
  for (uint32_t p0 = 0; p0 < nfull; p0 += 64 * U) {
    u32x4 va[NI][U], vb[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      if (F & kSrc) vb[u] = (p < nfull) ? ld16<kNT>(rsrc_, p * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    if (F & kRecv) {
      // all 4U lines of the lane (of every input) are loaded, then polled
      // together: one round trip per iteration however many packets
      uint64_t ln[NI][U][4];
#pragma unroll
      for (int i = 0; i < NI; i++)
#pragma unroll
        for (int u = 0; u < U; u++) {
          const uint32_t p = p0 + u * 64 + L.lane;
#pragma unroll
          for (int q = 0; q < 4; q++) ln[i][u][q] = (p < nfull) ? ld_relaxed(lin[i] + ll_line_index(p, q)) : ll_line(0, fin);
        }
      L.w.start();
      while (true) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
          for (int u = 0; u < U; u++)
#pragma unroll
            for (int q = 0; q < 4; q++) ok = ok && ll_ready(ln[i][u][q], fin);
        if (__all(ok)) break;
        if (!L.w.idle()) return false;
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
          for (int u = 0; u < U; u++) {
            const uint32_t p = p0 + u * 64 + L.lane;
#pragma unroll
            for (int q = 0; q < 4; q++)
              if (!ll_ready(ln[i][u][q], fin)) ln[i][u][q] = ld_relaxed(lin[i] + ll_line_index(p, q));
          }
      }
#pragma unroll
      for (int i = 0; i < NI; i++)
#pragma unroll
        for (int u = 0; u < U; u++)
          va[i][u] = u32x4{(uint32_t)ln[i][u][0], (uint32_t)ln[i][u][1], (uint32_t)ln[i][u][2], (uint32_t)ln[i][u][3]};
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      if (p >= nfull) continue;
      const u32x4 r = combine<E, OP, F>(va[0][u], va[NI - 1][u], vb[u], a.nranks);
      if (F & kSend) ll_send4(lout, p, r, fout);
      if (F & kSend2) ll_send4(lout2, p, r, fout);
      if (F & kDst) st16<kNT>(r, rdst, p * 16);
    }
  }
  bool failed = false;
#pragma unroll 1
  for (uint32_t p = nfull + L.lane; p < npk; p += 64) {
    const uint32_t off = p * 16, nb = min(16u, nbytes - off);
    u32x4 x[NI], y = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NI; i++) x[i] = y;
    if (F & kSrc) y = ld_part<E, kNT>(rsrc_, off, nb);
    if (F & kRecv) {
#pragma unroll
      for (int i = 0; i < NI; i++) {
        uint64_t ln[4];
        if (!ll_recv4(L.w, lin[i], p, true, fin, ln)) { failed = true; break; }
        x[i] = u32x4{(uint32_t)ln[0], (uint32_t)ln[1], (uint32_t)ln[2], (uint32_t)ln[3]};
      }
      if (failed) break;
    }
    const u32x4 r = combine<E, OP, F>(x[0], x[NI - 1], y, a.nranks);
    if (F & kSend) ll_send4(lout, p, r, fout);
    if (F & kSend2) ll_send4(lout2, p, r, fout);
    if (F & kDst) st_part<E, kNT>(r, rdst, off, nb);
  }
  if (__any(failed)) return false;
  if (F & kSend) L.sstep++;
  if (F & kRecv) release_slot<F>(L);
  return true;
}

// --- LL128: 128-byte lines, 120 data bytes + 8-byte flag -------------------
// Every line carries its flag (the step number) in bytes 120..127.  gfx950
// does not promise that a 128-byte line stored by 8 lanes becomes visible at
// once (the pages rely on NVLink for that), so visibility is ordered per
// batch instead: the producer stores the batch's data (whole lines with
// their flags in one full-line store), waits until those stores have
// completed, and only then stores the flag of the batch's last line; the
// consumer waits for that one flag, which orders every line of the batch,
// and then reads the data.  A batch is one FIFO slice (up to a slot of 256
// lines).  Data moves in rows of 8 lines, one 16-byte packet per lane: row r
// covers lines 8r .. 8r + 7, lane l takes line 8r + l / 8, column l % 8
// (columns 0..6: data bytes 16c .. 16c + 15; column 7 holds data bytes
// 112..119 and the flag).
constexpr uint32_t kLL128Batch = kLL128SlotLines;
constexpr int kLL128FlagsPerLane = (int)(kLL128Batch / 64);

// Rows of whole lines (all 120 data bytes inside the part, 16-byte aligned
// user buffers): every lane moves one 16-byte packet per row with one load
// and one store width.  Column 7 reads the line's last 16 data bytes
// (104..119) instead of its 8, so it shares bytes 104..111 with column 6;
// both lanes compute them from the same inputs and store the same values to
// the user buffer, and all of an iteration's loads complete before any of
// its stores, so this holds in place too.  Towards the FIFO, column 7 stores
// bytes 112..127 of the line: its 8 data bytes and the line's flag, so each
// line leaves in one full 128-byte store.  (The batch's last line never
// goes this way: its flag is stored only once all of the batch's data stores
// have completed, and that one flag is what a consumer waits for.)
// The resources end at the last whole line (FIFO: lim lines of 128 bytes,
// user: lim lines of 120), so the lanes of a row past it read zeros and their
// stores are dropped by the range check: no per-lane condition anywhere, and
// all of an iteration's loads are in flight together.
template <int F>
constexpr int ll128_rows() { return (F & kRecv2) ? kLL128WholeRows / 2 : kLL128WholeRows; }

template <class E, int OP, int F, int NO>
__device__ __forceinline__ void ll128_rows_iter(const rsrc_t (&win)[2], const rsrc_t (&wout)[2], rsrc_t wsrc,
                                                rsrc_t wdst, uint32_t line0, int lane, int nranks, uint64_t flag) {
  constexpr int R = ll128_rows<F>();
  const bool c7 = (lane & 7) == 7;
  const uint32_t coff = c7 ? 104u : (uint32_t)(lane & 7) * 16u;
  const uint32_t soff = c7 ? 112u : coff;   // FIFO store offset in the line
  const uint32_t lrow = (uint32_t)(lane >> 3);
  u32x4 va[R], va2[R], vb[R];
#pragma unroll
  for (int u = 0; u < R; u++) {
    const uint32_t line = line0 + 8 * u + lrow;
    if (F & kRecv) va[u] = ld16<kSC1>(win[0], line * 128 + coff);
    if (F & kRecv2) va2[u] = ld16<kSC1>(win[1], line * 128 + coff);
    if (F & kSrc) vb[u] = ld16<kNT>(wsrc, line * 120 + coff);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < R; u++) {
    const uint32_t line = line0 + 8 * u + lrow;
    const u32x4 r = combine<E, OP, F>(va[u], va2[u], vb[u], nranks);
    if (F & kSend) {
      const u32x4 w = c7 ? u32x4{r.z, r.w, (uint32_t)flag, (uint32_t)(flag >> 32)} : r;
#pragma unroll
      for (int o = 0; o < NO; o++) st16<kSC1>(w, wout[o], line * 128 + soff);
    }
    if (F & kDst) st16<kNT>(r, wdst, line * 120 + coff);
  }
}

// Lines [l0, l1) packet by packet: the batch's last line, and every line
// when a user buffer is not 16-byte aligned (then element-wise on the user
// side, as is a packet that the part ends inside).  Column 7 moves its 8 data
// bytes only; the flags of these lines are stored after the batch's data.
template <class E, int OP, int F, int NO>
__device__ __forceinline__ void ll128_packets(const rsrc_t (&rin)[2], const rsrc_t (&rout)[2], rsrc_t rsrc_,
                                              rsrc_t rdst, uint32_t nbytes, int vec, uint32_t l0, uint32_t l1,
                                              int lane, int nranks) {
#pragma unroll 1
  for (uint32_t p = l0 * 8 + (uint32_t)lane; p < l1 * 8; p += 64) {
    const uint32_t line = p >> 3, col = p & 7;
    const uint32_t uoff = line * 120 + col * 16;
    if (uoff >= nbytes) continue;
    const uint32_t psize = col == 7 ? 8u : 16u;
    const uint32_t nb = min(psize, nbytes - uoff);
    const bool whole = vec && nb == psize;
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, x2 = x, y = x;
    if (F & kRecv) x = col == 7 ? ld8<kSC1>(rin[0], line * 128 + 112) : ld16<kSC1>(rin[0], line * 128 + col * 16);
    if (F & kRecv2) x2 = col == 7 ? ld8<kSC1>(rin[1], line * 128 + 112) : ld16<kSC1>(rin[1], line * 128 + col * 16);
    if (F & kSrc) {
      if (whole) y = col == 7 ? ld8<kNT>(rsrc_, uoff) : ld16<kNT>(rsrc_, uoff);
      else y = ld_part<E, kNT>(rsrc_, uoff, nb);
    }
    const u32x4 r = combine<E, OP, F>(x, x2, y, nranks);
    if (F & kSend) {
#pragma unroll
      for (int o = 0; o < NO; o++) {
        if (col == 7) st8<kSC1>(r, rout[o], line * 128 + 112);
        else st16<kSC1>(r, rout[o], line * 128 + col * 16);
      }
    }
    if (F & kDst) {
      if (whole) {
        if (col == 7) st8<kNT>(r, rdst, uoff);
        else st16<kNT>(r, rdst, uoff);
      } else {
        st_part<E, kNT>(r, rdst, uoff, nb);
      }
    }
  }
}

template <class E, int OP, int F>
__device__ __forceinline__ bool slice_ll128(Lane& L, uint64_t es0, uint64_t ed0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  const uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
  if (!wait_outputs<F>(L)) return false;
  constexpr int NI = (F & kRecv2) ? 2 : 1;   // inputs
  constexpr int NO = (F & kSend2) ? 2 : 1;   // outputs
  constexpr uint32_t RL = 8 * ll128_rows<F>();   // lines per iteration of whole rows
  const uint64_t fin = a.base + L.rstep + 1;
  const uint64_t fout = a.base + L.sstep + 1;
  const uint64_t rslot = (L.rstep & (a.depth - 1)) * kLL128SlotBytes;
  const uint64_t sslot = (L.sstep & (a.depth - 1)) * kLL128SlotBytes;
  char* sin[2] = {L.in[0].fifo + rslot, L.in[NI - 1].fifo + rslot};
  char* sout[2] = {L.out[0].fifo + sslot, L.out[NO - 1].fifo + sslot};
  const rsrc_t rin[2] = {make_rsrc(sin[0], kLL128SlotBytes), make_rsrc(sin[1], kLL128SlotBytes)};
  const rsrc_t rout[2] = {make_rsrc(sout[0], kLL128SlotBytes), make_rsrc(sout[1], kLL128SlotBytes)};
  const char* src = L.src + es0 * sizeof(typename E::T);
  char* dst = L.dst + ed0 * sizeof(typename E::T);
  const rsrc_t rsrc_ = make_rsrc(src, nbytes);
  const rsrc_t rdst = make_rsrc(dst, nbytes);
  const uint32_t nlines = (nbytes + 119) / 120;
  // lines with all 120 data bytes in the part go in whole rows
  const uint32_t whole = a.vec_ok ? nbytes / 120 : 0;
  if ((F & kRecv) && L.cap) L.zbytes = max(L.zbytes, nlines * 128u);   // slot bytes read (see finish_input)
  for (uint32_t b0 = 0; b0 < nlines; b0 += kLL128Batch) {
    const uint32_t b1 = min(nlines, b0 + kLL128Batch);
    if (F & kRecv) {
      // Flag first, then data.  The producer stores the flag of the batch's
      // last line only after all of the batch's data stores have completed,
      // so once seen it orders every line of the batch: the wavefront waits
      // for that one flag (one line per poll for the whole wavefront) and
      // then reads the data.
      const uint64_t* lp[NI];
#pragma unroll
      for (int i = 0; i < NI; i++) lp[i] = (const uint64_t*)(sin[i] + (size_t)(b1 - 1) * 128 + 120);
      L.w.start();
      while (true) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NI; i++) ok = ok && ld_relaxed(lp[i]) == fin;
        if (__all(ok)) break;
        if (!L.w.idle()) return false;
      }
      compiler_fence();
    }
    // whole lines of the batch but its last: [b0, bw) go by rows
    const uint32_t bw = min(b1 - 1, max(b0, whole));
    if (bw > b0) {
      const rsrc_t win[2] = {make_rsrc(sin[0], bw * 128), make_rsrc(sin[1], bw * 128)};
      const rsrc_t wout[2] = {make_rsrc(sout[0], bw * 128), make_rsrc(sout[1], bw * 128)};
      const rsrc_t wsrc = make_rsrc(src, bw * 120);
      const rsrc_t wdst = make_rsrc(dst, bw * 120);
      for (uint32_t l0 = b0; l0 < bw; l0 += RL)
        ll128_rows_iter<E, OP, F, NO>(win, wout, wsrc, wdst, l0, L.lane, a.nranks, fout);
    }
    // the rest of the batch (its last line, and every line of unaligned
    // buffers): packet by packet
    ll128_packets<E, OP, F, NO>(rin, rout, rsrc_, rdst, nbytes, a.vec_ok, bw, b1, L.lane, a.nranks);
    if (F & kSend) {
      // all data of the batch is visible before the flags written now, those
      // of the lines that went packet by packet: the batch's last line
      // among them (the whole rows wrote their lines' flags with the data)
      wait_mem();
#pragma unroll
      for (int o = 0; o < NO; o++)
#pragma unroll
        for (int j = 0; j < kLL128FlagsPerLane; j++) {
          const uint32_t line = bw + 64 * j + L.lane;
          if (line < b1) st_relaxed((uint64_t*)(sout[o] + (size_t)line * 128 + 120), fout);
        }
    }
  }
  if (F & kSend) L.sstep++;
  if (F & kRecv) release_slot<F>(L);
  return true;
}

// --- small slices: at most one 16-byte packet per lane ---------------------
// Used when every lane part of the call is at most 1 KiB and all user
// buffers are 16-byte aligned: the sizes where a ring step's time is mostly
// the instructions of the step itself, so the code is straight-line.  Lane p
// handles packet p; a lane past the last packet points its accesses just past
// the buffer resources (LL: one per line column of the interleaved slot), so
// its loads read zeros and its stores are dropped by the range check.  The
// lane of a ragged last packet goes element-wise on the user side.
template <class E>
__device__ __forceinline__ u32x4 small_user_load(const Lane& L, uint64_t soff, uint32_t nbytes) {
  const uint32_t nfull = nbytes / 16, p = (uint32_t)L.lane;
  u32x4 v = ld16<kNT>(make_rsrc(L.src + soff, nfull * 16), p * 16);
  if (nfull * 16 < nbytes && p == nfull)
    v = ld_part<E, kNT>(make_rsrc(L.src + soff, nbytes), p * 16, nbytes - p * 16);
  return v;
}

template <class E>
__device__ __forceinline__ void small_user_store(const Lane& L, uint64_t doff, uint32_t nbytes, u32x4 v) {
  const uint32_t nfull = nbytes / 16, p = (uint32_t)L.lane;
  st16<kNT>(v, make_rsrc(L.dst + doff, nfull * 16), p * 16);
  if (nfull * 16 < nbytes && p == nfull)
    st_part<E, kNT>(v, make_rsrc(L.dst + doff, nbytes), p * 16, nbytes - p * 16);
}

template <class E, int OP, int F>
__device__ __forceinline__ bool slice_ll_small(Lane& L, uint64_t es0, uint64_t ed0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  const uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
  if (!wait_outputs<F>(L)) return false;
  constexpr int NI = (F & kRecv2) ? 2 : 1;   // inputs
  constexpr int NO = (F & kSend2) ? 2 : 1;   // outputs
  const uint32_t fin = (uint32_t)(a.base + L.rstep + 1);
  const uint32_t fout = (uint32_t)(a.base + L.sstep + 1);
  const uint64_t soff = es0 * sizeof(typename E::T), doff = ed0 * sizeof(typename E::T);
  const uint32_t npk = (nbytes + 15) / 16, p = (uint32_t)L.lane;
  const bool act = p < npk;
  if (npk == 0) {
    // an empty slice (a chunk past the end of a short buffer) moves and
    // polls no line; it still takes its step on both sides and frees its
    // input slot, so that the heads keep counting every step
    if (F & kSend) L.sstep++;
    if (F & kRecv) release_slot<F>(L);
    return true;
  }
  if ((F & kRecv) && L.cap) L.zbytes = max(L.zbytes, ll_prefix_bytes(npk));   // slot bytes read (see finish_input)
  u32x4 va[NI], vb = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < NI; i++) va[i] = vb;
  if (F & kSrc) vb = small_user_load<E>(L, soff, nbytes);
  if (F & kRecv) {
    // one resource per line column q, holding lines 64 q .. 64 q + npk - 1
    // (lanes past the last packet read zeros without a memory access)
    rsrc_t ri[NI][4];
    uint64_t ln[2][NI][4];
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        ri[i][q] = make_rsrc(L.in[i].fifo + (L.rstep & (a.depth - 1)) * kLLSlotBytes + ll_line_index(0, q) * 8,
                             npk * 8);
    // Two polls of the packet's lines in flight: each round waits for the
    // older one only and re-issues it, so a line that lands is seen about
    // half a load round trip sooner than with one poll at a time.  Flags only
    // move forward within the call, so either poll alone is a valid view.
#pragma unroll
    for (int k = 0; k < 2; k++)
#pragma unroll
      for (int i = 0; i < NI; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) ln[k][i][q] = ll_load(ri[i][q], p * 8);
    auto ready = [&](const uint64_t (&x)[NI][4]) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < NI; i++)
        ok = ok && (!act || (ll_ready(x[i][0], fin) && ll_ready(x[i][1], fin) && ll_ready(x[i][2], fin) &&
                             ll_ready(x[i][3], fin)));
      return __all(ok);
    };
    L.w.start();
    int k = 0;
    while (true) {
      if (ready(ln[0])) break;
      if (!L.w.idle()) return false;
#pragma unroll
      for (int i = 0; i < NI; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) ln[0][i][q] = ll_load(ri[i][q], p * 8);
      if (ready(ln[1])) {
        k = 1;
        break;
      }
      if (!L.w.idle()) return false;
#pragma unroll
      for (int i = 0; i < NI; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) ln[1][i][q] = ll_load(ri[i][q], p * 8);
    }
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const uint64_t* x = k ? ln[1][i] : ln[0][i];
      va[i] = u32x4{(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
    }
  }
  const u32x4 r = combine<E, OP, F>(va[0], va[NI - 1], vb, a.nranks);
  if (F & kSend) {
#pragma unroll
    for (int o = 0; o < NO; o++) {
      char* so = L.out[o].fifo + (L.sstep & (a.depth - 1)) * kLLSlotBytes;
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int q = 0; q < 4; q++) ll_store(make_rsrc(so + ll_line_index(0, q) * 8, npk * 8), p * 8, w[q], fout);
    }
    L.sstep++;
  }
  if (F & kDst) small_user_store<E>(L, doff, nbytes, r);
  if (F & kRecv) release_slot<F>(L);
  return true;
}

template <class E, int OP, int F>
__device__ __forceinline__ bool slice_simple_small(Lane& L, uint64_t es0, uint64_t ed0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  const uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
  if (!wait_inputs<F>(L) || !wait_outputs<F>(L)) return false;
  const uint64_t soff = es0 * sizeof(typename E::T), doff = ed0 * sizeof(typename E::T);
  const uint32_t npk = (nbytes + 15) / 16, p = (uint32_t)L.lane;
  const uint64_t rslot = (L.rstep & (a.depth - 1)) * kSimpleSlotBytes;
  const uint64_t sslot = (L.sstep & (a.depth - 1)) * kSimpleSlotBytes;
  u32x4 va = u32x4{0u, 0u, 0u, 0u}, va2 = va, vb = va;
  if (F & kRecv) va = ld16<kSC1>(make_rsrc(L.in[0].fifo + rslot, npk * 16), p * 16);
  if (F & kRecv2) va2 = ld16<kSC1>(make_rsrc(L.in[1].fifo + rslot, npk * 16), p * 16);
  if (F & kSrc) vb = small_user_load<E>(L, soff, nbytes);
  const u32x4 r = combine<E, OP, F>(va, va2, vb, a.nranks);
  if (F & kSend) st16<kSC1>(r, make_rsrc(L.out[0].fifo + sslot, npk * 16), p * 16);
  if (F & kSend2) st16<kSC1>(r, make_rsrc(L.out[1].fifo + sslot, npk * 16), p * 16);
  if (F & kDst) small_user_store<E>(L, doff, nbytes, r);
  if (F & kSend) publish_tails<F>(L);
  if (F & kRecv) release_slot<F>(L);
  return true;
}

// --- direct: the successor's receive buffer instead of a FIFO -------------
// The pages' "direct" primitives read and write the peer's user buffer
// without a staging FIFO ([ARCH] §九.4).  Here ring index i writes each
// outgoing slice into its successor's receive buffer at the slice's own
// element offset and publishes the tail; the successor reads it there (kRecv
// = read own receive buffer), folds in its own input and writes the result
// on into its successor's buffer (kSend), or keeps it (kDst).  Every slice
// has its own place, so no slot is reused and no head counter is needed: a
// partial result in a receive buffer is overwritten only by the final value
// of the same chunk, which can only arrive after the owner has read the
// partial and passed it on.  Only valid out of place (a partial result would
// otherwise overwrite the receiver's own input).
template <class E, int OP, int F>
__device__ __forceinline__ bool slice_direct(Lane& L, uint64_t e0, uint32_t nelem) {
  const KernelArgs& a = *L.a;
  const uint32_t nbytes = nelem * (uint32_t)sizeof(typename E::T);
  if ((F & kRecv) && !wait_ge(L.w, L.in[0].tail, a.base + L.rstep + 1, L.tail_seen[0])) return false;
  const uint64_t off = e0 * sizeof(typename E::T);
  rsrc_t rin = make_rsrc(L.dst + off, nbytes);     // own receive buffer, written by the predecessor
  rsrc_t rpeer = make_rsrc(L.peer + off, nbytes);  // the successor's receive buffer
  rsrc_t rsrc_ = make_rsrc(L.src + off, nbytes);
  rsrc_t rdst = rin;
  const uint32_t npk = (nbytes + 15) / 16;
  const uint32_t nfull = a.vec_ok ? nbytes / 16 : 0;
  // whole groups without per-lane conditions, as in slice_simple (half the
  // unroll for the division of an average)
  constexpr int U = (F & kPost) ? kUnroll / 2 : kUnroll;
  const uint32_t nmain = nfull - nfull % (64u * U);
  for (uint32_t p0 = 0; p0 < nmain; p0 += 64 * U) {
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t o = (p0 + u * 64 + L.lane) * 16;
      if (F & kRecv) va[u] = ld16<kSC1>(rin, o);
      if (F & kSrc) vb[u] = ld16<kNT>(rsrc_, o);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t o = (p0 + u * 64 + L.lane) * 16;
      const u32x4 r = combine<E, OP, F>(va[u], va[u], vb[u], a.nranks);
      if (F & kSend) st16<kSC1>(r, rpeer, o);
      if (F & kDst) st16<kNT>(r, rdst, o);
    }
  }
  for (uint32_t p0 = nmain; p0 < nfull; p0 += 64 * U) {
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      const bool in = p < nfull;
      if (F & kRecv) va[u] = in ? ld16<kSC1>(rin, p * 16) : u32x4{0u, 0u, 0u, 0u};
      if (F & kSrc) vb[u] = in ? ld16<kNT>(rsrc_, p * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t p = p0 + u * 64 + L.lane;
      if (p >= nfull) continue;
      const u32x4 r = combine<E, OP, F>(va[u], va[u], vb[u], a.nranks);
      if (F & kSend) st16<kSC1>(r, rpeer, p * 16);
      if (F & kDst) st16<kNT>(r, rdst, p * 16);
    }
  }
#pragma unroll 1
  for (uint32_t p = nfull + L.lane; p < npk; p += 64) {
    const uint32_t o = p * 16, nb = min(16u, nbytes - o);
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
    if (F & kRecv) x = ld_part<E, kSC1>(rin, o, nb);
    if (F & kSrc) y = ld_part<E, kNT>(rsrc_, o, nb);
    const u32x4 r = combine<E, OP, F>(x, x, y, a.nranks);
    if (F & kSend) st_part<E, kSC1>(r, rpeer, o, nb);
    if (F & kDst) st_part<E, kNT>(r, rdst, o, nb);
  }
  if (F & kSend) publish_tails<F>(L);
  if (F & kRecv) L.rstep++;
  return true;
}

// A primitive of the direct form over the lane's part of one chunk, in
// slices of one Simple slot (the tail's granularity).  A part the receiver
// does not need to read (the last stage: the data is already in its buffer)
// only advances its step count.
template <class E, int OP, int F>
__device__ __forceinline__ bool primitive_direct(Lane& L, uint64_t e0, uint64_t nelem) {
  const uint64_t cap = slot_elems(kSimple, sizeof(typename E::T));
  for (uint64_t j = 0; j < nelem; j += cap) {
    const uint32_t m = (uint32_t)min_u64(cap, nelem - j);
    if (F == kRecv) {
      L.rstep++;
      continue;
    }
    if (!slice_direct<E, OP, F>(L, e0 + j, m)) return false;
  }
  return true;
}

// --- a primitive over the lane's part of one chunk ------------------------
// es0 / ed0: element offsets of the part in the source and destination user
// buffers (equal in the AllReduce; block-relative in its two halves).
template <class E, int OP, int PROTO, int F, bool SMALL>
__device__ __forceinline__ bool primitive(Lane& L, uint64_t es0, uint64_t ed0, uint64_t nelem) {
  if constexpr (SMALL) {
    // the host launches this form only for lane parts of at most 1 KiB
    if (nelem * sizeof(typename E::T) > kSmallSliceBytes) {
      record_error(*L.a, kErrInternal);
      return false;
    }
    if (nelem == 0) return true;
    if (PROTO == kLL) return slice_ll_small<E, OP, F>(L, es0, ed0, (uint32_t)nelem);
    return slice_simple_small<E, OP, F>(L, es0, ed0, (uint32_t)nelem);
  }
  const uint64_t cap = slot_elems(PROTO, sizeof(typename E::T));
  // The host plans parts of at most half the FIFO depth; a larger one could
  // deadlock the ring, so refuse it instead.
  if (nelem > (uint64_t)(L.a->depth / 2) * cap) {
    record_error(*L.a, kErrInternal);
    return false;
  }
  for (uint64_t j = 0; j < nelem; j += cap) {
    uint32_t m = (uint32_t)min_u64(cap, nelem - j);
    bool ok;
    if (PROTO == kSimple) ok = slice_simple<E, OP, F>(L, es0 + j, ed0 + j, m);
    else if (PROTO == kLL) ok = slice_ll<E, OP, F>(L, es0 + j, ed0 + j, m);
    else ok = slice_ll128<E, OP, F>(L, es0 + j, ed0 + j, m);
    if (!ok) return false;
  }
  return true;
}

// One launch of a ring collective: every (ring index, channel, lane)
// wavefront of every virtual rank.  COLL: kAllReduce (2n-1 stages per loop),
// kReduceScatter or kAllGather (n stages per loop, whole blocks by rank).
template <class E, int OP, int PROTO, bool SMALL, int COLL>
__device__ __forceinline__ void ring_body(const KernelArgs& a, bool cap) {
  static_assert(!SMALL || PROTO != kLL128, "no small-slice form of LL128");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps lane-derived values scalar
  int group, ri;                               // (channel, lane block), ring index
  block_group(blockIdx.x, a.nranks, a.xcd_major, &group, &ri);
  const int lane_blocks = a.lanes / a.lanes_per_block;
  if (group >= a.nchannels * lane_blocks) return;   // XCD-major padding
  const int c = group / lane_blocks;
  const int l = (group % lane_blocks) * a.lanes_per_block + wave;
  if (ri == a.skip_ring_index) return;
  const int n = a.nranks;
  const uint32_t es = sizeof(typename E::T);

  Lane L;
  L.a = &a;
  L.w.a = &a;
  L.lane = threadIdx.x & 63;
  L.cap = cap;
  L.zbytes = 0;
  L.sstep = 0;
  L.rstep = 0;
  L.tail_seen[0] = L.tail_seen[1] = 0;   // below any value a wait of this call asks for
  L.head_seen[0] = L.head_seen[1] = 0;
  L.in[0] = conn_at<PROTO>(a, conn_index(c, ri, l, n, a.lanes));
  L.out[0] = conn_at<PROTO>(a, conn_index(c, (ri + 1) % n, l, n, a.lanes));
  L.src = a.send[ri];
  L.dst = a.recv[ri];
  L.peer = a.recv[(ri + 1) % n];

  uint64_t lo, hi;
  channel_bounds(a.count, a.per_channel, c, &lo, &hi);
  const uint64_t len = hi - lo;
  if constexpr (COLL == kAllReduce && PROTO == kSimple && !SMALL) {
    if (a.direct) {
      const uint64_t loop = (uint64_t)n * a.chunk_elems;
      for (uint64_t off = 0; off < len; off += loop) {
        const uint64_t rem = len - off;
        const uint64_t cur = loop_chunk(len, off, n, a.chunk_elems, es);
        const uint64_t part = lane_part(cur, a.lanes, es, PROTO);
        for (int s = 0; s <= 2 * n - 2; s++) {
          const int k = stage_chunk(ri, s, n);
          uint64_t ks, kl, ls, ll;
          chunk_bounds(rem, cur, k, &ks, &kl);
          lane_bounds(kl, part, l, &ls, &ll);
          const uint64_t e0 = lo + off + ks + ls;
          bool ok;
          if (s == 0) ok = primitive_direct<E, OP, kSrc | kSend>(L, e0, ll);
          else if (s <= n - 2) ok = primitive_direct<E, OP, kRecv | kSrc | kSend>(L, e0, ll);
          else if (s == n - 1) ok = primitive_direct<E, OP, kRecv | kSrc | kSend | kDst | post_flag<OP>()>(L, e0, ll);
          else if (s <= 2 * n - 3) ok = primitive_direct<E, OP, kRecv | kSend>(L, e0, ll);
          else ok = primitive_direct<E, OP, kRecv>(L, e0, ll);
          if (!ok) return;
        }
      }
      return;
    }
  }
  if constexpr (COLL == kAllReduce) {
    const uint64_t loop = (uint64_t)n * a.chunk_elems;
    for (uint64_t off = 0; off < len; off += loop) {
      const uint64_t rem = len - off;
      const uint64_t cur = loop_chunk(len, off, n, a.chunk_elems, es);
      const uint64_t part = lane_part(cur, a.lanes, es, PROTO);
      for (int s = 0; s <= 2 * n - 2; s++) {
        const int k = stage_chunk(ri, s, n);
        uint64_t ks, kl, ls, ll;
        chunk_bounds(rem, cur, k, &ks, &kl);
        lane_bounds(kl, part, l, &ls, &ll);
        const uint64_t e0 = lo + off + ks + ls;
        bool ok;
        if (s == 0) ok = primitive<E, OP, PROTO, kSrc | kSend, SMALL>(L, e0, e0, ll);
        else if (s <= n - 2) ok = primitive<E, OP, PROTO, kRecv | kSrc | kSend, SMALL>(L, e0, e0, ll);
        else if (s == n - 1) ok = primitive<E, OP, PROTO, kRecv | kSrc | kSend | kDst | post_flag<OP>(), SMALL>(L, e0, e0, ll);
        else if (s <= 2 * n - 3) ok = primitive<E, OP, PROTO, kRecv | kSend | kDst, SMALL>(L, e0, e0, ll);
        else ok = primitive<E, OP, PROTO, kRecv | kDst, SMALL>(L, e0, e0, ll);
        if (!ok) return;
      }
    }
  } else {
    // The halves: a.count is the block length; a loop takes up to one chunk
    // of every block, and the block of rank q starts at q * a.count.
    for (uint64_t off = 0; off < len; off += a.chunk_elems) {
      const uint64_t cur = min_u64(a.chunk_elems, len - off);
      const uint64_t part = lane_part(cur, a.lanes, es, PROTO);
      uint64_t ls, ll;
      lane_bounds(cur, part, l, &ls, &ll);
      const uint64_t pos = lo + off + ls;           // element offset inside a block
      for (int s = 0; s <= n - 1; s++) {
        const int k = COLL == kReduceScatter ? stage_chunk(ri, s, n) : (ri - s + n) % n;
        const uint64_t blk = (uint64_t)a.rank_of[k] * a.count + pos;
        bool ok;
        if (COLL == kReduceScatter) {
          if (s == 0) ok = primitive<E, OP, PROTO, kSrc | kSend, SMALL>(L, blk, 0, ll);
          else if (s <= n - 2) ok = primitive<E, OP, PROTO, kRecv | kSrc | kSend, SMALL>(L, blk, 0, ll);
          else ok = primitive<E, OP, PROTO, kRecv | kSrc | kDst | post_flag<OP>(), SMALL>(L, blk, pos, ll);
        } else {
          if (s == 0) ok = primitive<E, OP, PROTO, kSrc | kSend | kDst, SMALL>(L, pos, blk, ll);
          else if (s <= n - 2) ok = primitive<E, OP, PROTO, kRecv | kSend | kDst, SMALL>(L, 0, blk, ll);
          else ok = primitive<E, OP, PROTO, kRecv | kDst, SMALL>(L, 0, blk, ll);
        }
        if (!ok) return;
      }
    }
  }
  if (cap) finish_input<PROTO>(L, L.in[0]);
}

// The Simple kernels are held to 128 VGPRs so that 16 wavefronts fit a CU
// (occupancy 4: the 4096-wavefront launches of large calls); none of them,
// eager or captured, needs scratch under that bound.  The line protocols (LL,
// LL128) keep their registers: LL's general form (131-134 VGPRs) would spill
// under it.
// CAP: the captured form (its own instances, so that the eager ones carry
// none of its code).
template <class E, int OP, int PROTO, bool SMALL, int COLL, bool CAP = false>
__global__ void __launch_bounds__(256, 4) ring_kernel(const KernelArgs a) {
  static_assert(PROTO == kSimple, "the line protocols run ring_kernel_lines");
  ring_body<E, OP, PROTO, SMALL, COLL>(a, CAP);
}
template <class E, int OP, int PROTO, bool SMALL, int COLL, bool CAP = false>
__global__ void __launch_bounds__(256) ring_kernel_lines(const KernelArgs a) {
  static_assert(PROTO != kSimple, "Simple runs ring_kernel");
  ring_body<E, OP, PROTO, SMALL, COLL>(a, CAP);
}
// The captured line kernels, held to occupancy 3 or more (at most 168
// VGPRs), the eager line kernels' lowest; they take 105-136 VGPRs, so the
// bound only keeps a later change from dropping them to 2.
template <class E, int OP, int PROTO, bool SMALL, int COLL>
__global__ void __launch_bounds__(256, 3) ring_kernel_lines_captured(const KernelArgs a) {
  static_assert(PROTO != kSimple, "Simple runs ring_kernel");
  ring_body<E, OP, PROTO, SMALL, COLL>(a, true);
}

// ----------------------------------------------------------------- tree
// One launch of the tree AllReduce over the double binary tree of
// [ARCH] §五.4 (channel c runs on tree c % 2): the reduce runs up the tree
// and the root's result is broadcast back down ([ARCH] §七.1 and §九.4,
// runTreeUpDown / runTreeSplit), with the up and down directions on separate
// wavefronts so that each chunk starts down as soon as the root has it.
// Per chunk of the channel, in lane parts as on the ring:
//   reduce role of v:    own input folded with child 0's, then child 1's
//                        partial result (each hop op(received, local)),
//                        sent to the parent (leaves: send only);
//   root:                the same fold, written to its output and sent to
//                        its children;
//   broadcast role of v: receives the result from the parent, writes its
//                        output and forwards it to its children.
// Every connection carries the same sequence of slices, so producer and
// consumer agree on step numbers as on the ring.
template <class E, int OP, int PROTO, bool SMALL, int F>
__device__ __forceinline__ bool tree_chunks(Lane& L, uint64_t lo, uint64_t len, int l, uint32_t es) {
  const KernelArgs& a = *L.a;
  for (uint64_t off = 0; off < len; off += a.chunk_elems) {
    const uint64_t cur = min_u64(a.chunk_elems, len - off);
    const uint64_t part = lane_part(cur, a.lanes, es, PROTO);
    uint64_t ls, ll;
    lane_bounds(cur, part, l, &ls, &ll);
    const uint64_t e0 = lo + off + ls;
    if (!primitive<E, OP, PROTO, F, SMALL>(L, e0, e0, ll)) return false;
  }
  return true;
}

// CAP: the captured form, as for the ring: steps from zero, every consumed
// flag and counter left at zero (a vertex resets the connections it receives
// on, the children's up connections or its parent's down connection).
template <class E, int OP, int PROTO, bool SMALL, bool CAP>
__device__ __forceinline__ void tree_body(const TreeArgs& ta) {
  static_assert(!SMALL || PROTO != kLL128, "no small-slice form of LL128");
  const KernelArgs& a = ta.k;
  const int n = a.nranks;
  const int R = tree_roles(n);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps lane-derived values scalar
  int group, role;
  block_group(blockIdx.x, R, a.xcd_major, &group, &role);
  const int lane_blocks = a.lanes / a.lanes_per_block;
  if (group >= a.nchannels * lane_blocks) return;   // XCD-major padding
  const int c = group / lane_blocks;
  const int l = (group % lane_blocks) * a.lanes_per_block + wave;
  const int t = c & 1;
  const int root = ta.root[t];
  const bool bcast = role >= n;
  int v = role;
  if (bcast) {
    v = role - n;
    if (v >= root) v++;
  }
  if (v == a.skip_ring_index) return;
  const uint32_t es = sizeof(typename E::T);

  Lane L;
  L.a = &a;
  L.w.a = &a;
  L.lane = threadIdx.x & 63;
  L.cap = CAP;
  L.zbytes = 0;
  L.sstep = 0;
  L.rstep = 0;
  L.tail_seen[0] = L.tail_seen[1] = 0;
  L.head_seen[0] = L.head_seen[1] = 0;
#ifdef RINGAR_ROLE_PROFILE
  L.w_in = L.w_out = L.n_sl = 0;
  const uint64_t tstart = wall_clock64();
#endif
  L.src = a.send[v];
  L.dst = a.recv[v];
  // present children in child-slot order: k0 first, then k1 (-1 = none);
  // an unused connection points at k0's so that it is still a valid address
  const int s0 = ta.child[t][0][v], s1 = ta.child[t][1][v];
  const int k0 = s0 >= 0 ? s0 : s1;
  const int k1 = s0 >= 0 ? s1 : -1;
  const int nk = (k0 >= 0 ? 1 : 0) + (k1 >= 0 ? 1 : 0);
  const int k0c = k0 >= 0 ? k0 : v, k1c = k1 >= 0 ? k1 : k0c;
  if (!bcast) {
    // inputs: the children's up connections
    L.in[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kUp, l, n, a.lanes));
    L.in[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kUp, l, n, a.lanes));
    if (v == root) {
      L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kDown, l, n, a.lanes));
      L.out[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kDown, l, n, a.lanes));
    } else {
      L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, v, kUp, l, n, a.lanes));
      L.out[1] = L.out[0];
    }
  } else {
    L.in[0] = conn_at<PROTO>(a, tree_conn_index(c, v, kDown, l, n, a.lanes));
    L.in[1] = L.in[0];
    L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kDown, l, n, a.lanes));
    L.out[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kDown, l, n, a.lanes));
  }

  uint64_t lo, hi;
  channel_bounds(a.count, a.per_channel, c, &lo, &hi);
  const uint64_t len = hi - lo;
  if (!bcast && v == root) {
    // (n >= 2, so the root has at least one child)
    constexpr int P = post_flag<OP>();
    if (nk == 1) tree_chunks<E, OP, PROTO, SMALL, kSrc | kRecv | kDst | kSend | P>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, SMALL, kSrc | kRecv | kRecv2 | kDst | kSend | kSend2 | P>(L, lo, len, l, es);
  } else if (!bcast) {
    if (nk == 0) tree_chunks<E, OP, PROTO, SMALL, kSrc | kSend>(L, lo, len, l, es);
    else if (nk == 1) tree_chunks<E, OP, PROTO, SMALL, kSrc | kRecv | kSend>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, SMALL, kSrc | kRecv | kRecv2 | kSend>(L, lo, len, l, es);
  } else {
    if (nk == 0) tree_chunks<E, OP, PROTO, SMALL, kRecv | kDst>(L, lo, len, l, es);
    else if (nk == 1) tree_chunks<E, OP, PROTO, SMALL, kRecv | kDst | kSend>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, SMALL, kRecv | kDst | kSend | kSend2>(L, lo, len, l, es);
  }
  if (CAP) {
    // only real inputs: a leaf's unused input slot points at its own output
    if (bcast || nk >= 1) finish_input<PROTO>(L, L.in[0]);
    if (!bcast && nk == 2) finish_input<PROTO>(L, L.in[1]);
  }
#ifdef RINGAR_ROLE_PROFILE
  if (PROTO == kSimple && !SMALL && !CAP && L.lane == 0) {
    const uint32_t id = blockIdx.x * (blockDim.x / 64) + wave;
    if (id < (uint32_t)kRoleProfileWaves) {
      unsigned long long* r = g_role_profile[id];
      r[0] = tstart;
      r[1] = wall_clock64();
      r[2] = L.w_in;
      r[3] = L.w_out;
      r[4] = L.n_sl;
      r[5] = (uint64_t)v | ((uint64_t)bcast << 8) | ((uint64_t)nk << 16) | ((uint64_t)(v == root) << 24);
      r[6] = (uint64_t)c;
      r[7] = (uint64_t)l;
    }
  }
#endif
}

// ----------------------------------------------------------------- split tree (Simple)
// The split form of the tree AllReduce: every role that moves four or more
// units of its channel per element (the root's reduce role, the reduce and
// broadcast roles of a vertex with two children) runs as two wavefronts,
// each on half of every slice, so that the roles that set the tree's pace
// have twice the loads in flight.  Its connections keep their slots; a
// split producer publishes each half's tail on a word of its own and a
// split consumer frees each half on a word of its own, and the other side
// waits for both.  Eager calls only (the plan never splits a captured call).
template <class E, int OP>
__device__ __forceinline__ void tree_body_split(const TreeArgs& ta) {
  constexpr int PROTO = kSimple;
  const KernelArgs& a = ta.k;
  const int n = a.nranks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int group, role;
  block_group(blockIdx.x, ta.nroles, a.xcd_major, &group, &role);
  const int lane_blocks = a.lanes / a.lanes_per_block;
  if (group >= a.nchannels * lane_blocks) return;   // XCD-major padding
  const int c = group / lane_blocks;
  const int l = (group % lane_blocks) * a.lanes_per_block + wave;
  const int t = c & 1;
  const int root = ta.root[t];
  const int entry = ta.role_of[t][role];
  const int v = entry & 63;
  const bool bcast = (entry >> 6) & 1;
  if (v == a.skip_ring_index) return;
  const uint32_t es = sizeof(typename E::T);

  Lane L;
  L.a = &a;
  L.w.a = &a;
  L.lane = threadIdx.x & 63;
  L.cap = false;
  L.zbytes = 0;
  L.sstep = 0;
  L.rstep = 0;
  L.tail_seen[0] = L.tail_seen[1] = 0;
  L.head_seen[0] = L.head_seen[1] = 0;
  L.tail2_seen[0] = L.tail2_seen[1] = 0;
  L.head2_seen[0] = L.head2_seen[1] = 0;
#ifdef RINGAR_ROLE_PROFILE
  L.w_in = L.w_out = L.n_sl = 0;
  const uint64_t tstart = wall_clock64();
#endif
  L.src = a.send[v];
  L.dst = a.recv[v];
  const int s0 = ta.child[t][0][v], s1 = ta.child[t][1][v];
  const int k0 = s0 >= 0 ? s0 : s1;
  const int k1 = s0 >= 0 ? s1 : -1;
  const int nk = (k0 >= 0 ? 1 : 0) + (k1 >= 0 ? 1 : 0);
  const int k0c = k0 >= 0 ? k0 : v, k1c = k1 >= 0 ? k1 : k0c;
  const SplitRole sr = tree_split_role(ta, t, v, bcast);
  L.my_split = sr.my_split;
  L.my_half = (entry >> 7) & 1;
  L.in_split[0] = sr.in_split[0];
  L.in_split[1] = sr.in_split[1];
  L.out_split[0] = sr.out_split[0];
  L.out_split[1] = sr.out_split[1];
  if (!bcast) {
    // inputs: the children's up connections, written by their reduce roles
    L.in[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kUp, l, n, a.lanes));
    L.in[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kUp, l, n, a.lanes));
    if (v == root) {
      // outputs: the children's down connections, read by their broadcast roles
      L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kDown, l, n, a.lanes));
      L.out[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kDown, l, n, a.lanes));
    } else {
      // output: the up connection to the parent, read by its reduce role
      L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, v, kUp, l, n, a.lanes));
      L.out[1] = L.out[0];
    }
  } else {
    // input: the down connection from the parent (its broadcast role, or the
    // root's reduce role); outputs: the children's down connections
    L.in[0] = conn_at<PROTO>(a, tree_conn_index(c, v, kDown, l, n, a.lanes));
    L.in[1] = L.in[0];
    L.out[0] = conn_at<PROTO>(a, tree_conn_index(c, k0c, kDown, l, n, a.lanes));
    L.out[1] = conn_at<PROTO>(a, tree_conn_index(c, k1c, kDown, l, n, a.lanes));
  }

  uint64_t lo, hi;
  channel_bounds(a.count, a.per_channel, c, &lo, &hi);
  const uint64_t len = hi - lo;
  constexpr int S = kSplit;
  if (!bcast && v == root) {
    constexpr int P = post_flag<OP>();
    if (nk == 1) tree_chunks<E, OP, PROTO, false, kSrc | kRecv | kDst | kSend | P | S>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, false, kSrc | kRecv | kRecv2 | kDst | kSend | kSend2 | P | S>(L, lo, len, l, es);
  } else if (!bcast) {
    if (nk == 0) tree_chunks<E, OP, PROTO, false, kSrc | kSend | S>(L, lo, len, l, es);
    else if (nk == 1) tree_chunks<E, OP, PROTO, false, kSrc | kRecv | kSend | S>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, false, kSrc | kRecv | kRecv2 | kSend | S>(L, lo, len, l, es);
  } else {
    if (nk == 0) tree_chunks<E, OP, PROTO, false, kRecv | kDst | S>(L, lo, len, l, es);
    else if (nk == 1) tree_chunks<E, OP, PROTO, false, kRecv | kDst | kSend | S>(L, lo, len, l, es);
    else tree_chunks<E, OP, PROTO, false, kRecv | kDst | kSend | kSend2 | S>(L, lo, len, l, es);
  }
#ifdef RINGAR_ROLE_PROFILE
  if (L.lane == 0) {
    const uint32_t id = blockIdx.x * (blockDim.x / 64) + wave;
    if (id < (uint32_t)kRoleProfileWaves) {
      unsigned long long* r = g_role_profile[id];
      r[0] = tstart;
      r[1] = wall_clock64();
      r[2] = L.w_in;
      r[3] = L.w_out;
      r[4] = L.n_sl;
      r[5] = (uint64_t)v | ((uint64_t)bcast << 8) | ((uint64_t)nk << 16) | ((uint64_t)(v == root) << 24) |
             ((uint64_t)L.my_split << 32) | ((uint64_t)L.my_half << 33);
      r[6] = (uint64_t)c;
      r[7] = (uint64_t)l;
    }
  }
#endif
}

// The tree's Simple kernels (both forms) carry the ring's launch bound (4
// workgroups of 256 per CU, so at most 128 VGPRs: the launches of large
// calls fill the GPU's 4096 wavefronts, which needs occupancy 4); the line
// protocols keep their registers.
template <class E, int OP, int PROTO, bool SMALL, bool CAP = false>
__global__ void __launch_bounds__(256, 4) tree_kernel_simple(const TreeArgs ta) {
  static_assert(PROTO == kSimple, "the line protocols run tree_kernel");
  tree_body<E, OP, PROTO, SMALL, CAP>(ta);
}
// The split form, an entry point of its own (its primitives carry kSplit).
template <class E, int OP>
__global__ void __launch_bounds__(256, 4) tree_kernel_split(const TreeArgs ta) {
  tree_body_split<E, OP>(ta);
}
template <class E, int OP, int PROTO, bool SMALL, bool CAP = false>
__global__ void __launch_bounds__(256) tree_kernel(const TreeArgs ta) {
  static_assert(PROTO != kSimple, "Simple runs tree_kernel_simple");
  tree_body<E, OP, PROTO, SMALL, CAP>(ta);
}
}  // namespace ringar
