/*
 * Ring AllReduce oracle: a plain, sequential, slow CPU model of the ring
 * AllReduce that NCCL runs on the device (reduce-scatter, then all-gather,
 * 2(n-1) ring steps per loop, each channel on its own contiguous range).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this file's library.  The product
 * library neither links nor calls it, and the two share no code, headers or
 * constants.
 *
 * Sources, cited by page title and section:
 *   [ARCH]  arganzheng.life, "NCCL architecture: topology, channels,
 *           algorithms and protocols" (Chinese; part 4 of the series).
 *   [BOOK]  aireadcode.com, "NCCL Source Code Deep Dive: A GPU Journey of One
 *           AllReduce" (English edition; the Japanese edition holds ch. 5-6).
 *
 * What is computed (plain reading of the pages, one decision per step):
 *   1. Channel split: each channel owns one contiguous range of the buffer
 *      ([BOOK] §2.2, channels split count/nChannels contiguously).  The pages
 *      leave remainder and alignment open; this oracle rounds the per-channel
 *      length up to whole 16-byte units, so trailing channels may be short or
 *      empty.
 *   2. Loops inside a channel: one loop covers nranks chunks of chunk_elems
 *      elements; the last, partial loop uses chunks of
 *      alignUp(ceil(rem / nranks), 16 B / elemSize) elements
 *      ([BOOK] §2.3, RingARAlgorithm::getNextSendAddr).
 *   3. Chunk visited at stage s by ring index i: (i + n - 1 - s) mod n
 *      ([BOOK] §2.3, chunkId formula).
 *   4. Primitive order per loop ([ARCH] §九.4, runRing): send;
 *      (n-2) x recvReduceSend; recvReduceCopySend (the chunk is final here);
 *      (n-2) x recvCopySend; recv.
 *   5. Arithmetic: op(received, local) per hop.  Integers wrap (two's
 *      complement).  fp16 and bf16 widen both operands exactly to fp32, apply
 *      the op in fp32 and round back to 16 bits to nearest-even on every hop.
 *      fp32 and fp64 use IEEE binary ops (no contraction; build with
 *      -ffp-contract=off).  min keeps the received value unless the local one
 *      is strictly smaller; max likewise with strictly larger.
 *
 * The stage simulation keeps one payload buffer per ring index: what that
 * ring index put into its successor's FIFO at the previous stage.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Codes private to this file; the Python wrapper maps names onto them. */
enum { OR_I8 = 0, OR_I32 = 1, OR_F16 = 2, OR_BF16 = 3, OR_F32 = 4, OR_F64 = 5 };
enum { OR_SUM = 0, OR_PROD = 1, OR_MIN = 2, OR_MAX = 3, OR_AVG = 4 };

static size_t elem_size(int dtype) {
  switch (dtype) {
    case OR_I8: return 1;
    case OR_I32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_F32: return 4;
    case OR_F64: return 8;
    default: return 0;
  }
}

static size_t div_up(size_t a, size_t b) { return (a + b - 1) / b; }
static size_t align_up(size_t a, size_t b) { return div_up(a, b) * b; }
static size_t min_sz(size_t a, size_t b) { return a < b ? a : b; }

/* ---------------------------------------------------------------------
 * 16-bit float formats, written from the IEEE-754 definitions.
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: the upper half of binary32: 1 sign, 8 exponent (bias 127),
 *           7 fraction bits.
 * Decoding is exact.  Encoding rounds to nearest, ties to even: the value is
 * divided by the spacing of the target format at its magnitude (a power of
 * two, so the division is exact in double), rounded to an integer with rint()
 * in the default rounding mode, and scaled back.
 * --------------------------------------------------------------------- */
static float f16_decode(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);       /* (1 + m/2^10) 2^(e-15) */
  return (float)(s ? -v : v);
}

static uint16_t f16_encode_rne(float f) {
  double v = f;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return sign | 0x7e00;
  int e;
  frexp(a, &e);                                     /* a in [2^(e-1), 2^e) */
  int ex = e - 1;
  double q = (a == 0.0 || ex < -14) ? ldexp(1.0, -24) : ldexp(1.0, ex - 10);
  double r = rint(a / q) * q;
  if (r >= 65536.0) return sign | 0x7c00;            /* beyond 65504 -> inf */
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
  frexp(r, &e);
  ex = e - 1;
  uint16_t mant = (uint16_t)(r / ldexp(1.0, ex - 10) - 1024.0);
  return sign | (uint16_t)((ex + 15) << 10) | mant;
}

static float bf16_decode(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 0xff, m = h & 0x7f;
  double v;
  if (e == 0) v = ldexp((double)m, -133);           /* subnormal: m * 2^-133 */
  else if (e == 255) v = m ? NAN : INFINITY;
  else v = ldexp((double)(128 + m), e - 134);       /* (1 + m/2^7) 2^(e-127) */
  return (float)(s ? -v : v);
}

static uint16_t bf16_encode_rne(float f) {
  double v = f;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return sign | 0x7fc0;
  int e;
  frexp(a, &e);
  int ex = e - 1;
  double q = (a == 0.0 || ex < -126) ? ldexp(1.0, -133) : ldexp(1.0, ex - 7);
  double r = rint(a / q) * q;
  if (r >= ldexp(1.0, 128)) return sign | 0x7f80;   /* beyond max -> inf */
  if (r < ldexp(1.0, -126)) return sign | (uint16_t)(r / ldexp(1.0, -133));
  frexp(r, &e);
  ex = e - 1;
  uint16_t mant = (uint16_t)(r / ldexp(1.0, ex - 7) - 128.0);
  return sign | (uint16_t)((ex + 127) << 7) | mant;
}

/* Exposed so the tests can pin the codecs against library conversions. */
float oracle_f16_to_f32(uint16_t h) { return f16_decode(h); }
uint16_t oracle_f32_to_f16(float f) { return f16_encode_rne(f); }
float oracle_bf16_to_f32(uint16_t h) { return bf16_decode(h); }
uint16_t oracle_f32_to_bf16(float f) { return bf16_encode_rne(f); }

/* ---------------------------------------------------------------------
 * One hop of the reduction: out[e] = op(recv[e], local[e]).
 * --------------------------------------------------------------------- */
static float op_f32(int op, float a, float b) {
  switch (op) {
    case OR_SUM: return a + b;
    case OR_PROD: return a * b;
    case OR_MIN: return (b < a) ? b : a;
    default: return (b > a) ? b : a;
  }
}

static double op_f64(int op, double a, double b) {
  switch (op) {
    case OR_SUM: return a + b;
    case OR_PROD: return a * b;
    case OR_MIN: return (b < a) ? b : a;
    default: return (b > a) ? b : a;
  }
}

static void combine(int dtype, int op, const void* recv, const void* local,
                    void* out, size_t len) {
  size_t e;
  switch (dtype) {
    case OR_I8: {
      const uint8_t* a = recv; const uint8_t* b = local; uint8_t* o = out;
      for (e = 0; e < len; e++) {
        int8_t sa = (int8_t)a[e], sb = (int8_t)b[e];
        switch (op) {
          case OR_SUM: o[e] = (uint8_t)(a[e] + b[e]); break;
          case OR_PROD: o[e] = (uint8_t)((unsigned)a[e] * (unsigned)b[e]); break;
          case OR_MIN: o[e] = (sb < sa) ? b[e] : a[e]; break;
          default: o[e] = (sb > sa) ? b[e] : a[e]; break;
        }
      }
      break;
    }
    case OR_I32: {
      const uint32_t* a = recv; const uint32_t* b = local; uint32_t* o = out;
      for (e = 0; e < len; e++) {
        int32_t sa = (int32_t)a[e], sb = (int32_t)b[e];
        switch (op) {
          case OR_SUM: o[e] = a[e] + b[e]; break;
          case OR_PROD: o[e] = a[e] * b[e]; break;
          case OR_MIN: o[e] = (sb < sa) ? b[e] : a[e]; break;
          default: o[e] = (sb > sa) ? b[e] : a[e]; break;
        }
      }
      break;
    }
    case OR_F16: {
      const uint16_t* a = recv; const uint16_t* b = local; uint16_t* o = out;
      for (e = 0; e < len; e++)
        o[e] = f16_encode_rne(op_f32(op, f16_decode(a[e]), f16_decode(b[e])));
      break;
    }
    case OR_BF16: {
      const uint16_t* a = recv; const uint16_t* b = local; uint16_t* o = out;
      for (e = 0; e < len; e++)
        o[e] = bf16_encode_rne(op_f32(op, bf16_decode(a[e]), bf16_decode(b[e])));
      break;
    }
    case OR_F32: {
      const float* a = recv; const float* b = local; float* o = out;
      for (e = 0; e < len; e++) o[e] = op_f32(op, a[e], b[e]);
      break;
    }
    default: {
      const double* a = recv; const double* b = local; double* o = out;
      for (e = 0; e < len; e++) o[e] = op_f64(op, a[e], b[e]);
      break;
    }
  }
}

/* ---------------------------------------------------------------------
 * The average.  [ARCH] §九.4 marks the step where a chunk becomes final
 * (recvReduceCopySend) with postOp=true; the pages say nothing more.
 * Reading: avg folds every hop like sum, and only the final value is divided
 * by the rank count, once, where the chunk becomes final; the quotient is
 * what is stored and forwarded.  Integers: signed division truncating toward
 * zero (C).  fp32 / fp64: one IEEE division.  fp16 / bf16: widen exactly to
 * fp32, divide in fp32, round to nearest-even (fp32 has more than twice the
 * 16-bit formats' precision plus two bits, so this is the correctly rounded
 * 16-bit quotient).
 * --------------------------------------------------------------------- */
static int hop_op(int op) { return op == OR_AVG ? OR_SUM : op; }

static void average(int dtype, void* buf, size_t len, int n) {
  size_t e;
  switch (dtype) {
    case OR_I8: {
      uint8_t* b = buf;
      for (e = 0; e < len; e++) b[e] = (uint8_t)(int8_t)((int)(int8_t)b[e] / n);
      break;
    }
    case OR_I32: {
      uint32_t* b = buf;
      for (e = 0; e < len; e++) b[e] = (uint32_t)((int32_t)b[e] / (int32_t)n);
      break;
    }
    case OR_F16: {
      uint16_t* b = buf;
      for (e = 0; e < len; e++) b[e] = f16_encode_rne(f16_decode(b[e]) / (float)n);
      break;
    }
    case OR_BF16: {
      uint16_t* b = buf;
      for (e = 0; e < len; e++) b[e] = bf16_encode_rne(bf16_decode(b[e]) / (float)n);
      break;
    }
    case OR_F32: {
      float* b = buf;
      for (e = 0; e < len; e++) b[e] = b[e] / (float)n;
      break;
    }
    default: {
      double* b = buf;
      for (e = 0; e < len; e++) b[e] = b[e] / (double)n;
      break;
    }
  }
}

/* ---------------------------------------------------------------------
 * Partition (steps 1-3 of the header).
 * --------------------------------------------------------------------- */

/* Channel c's element range [lo, hi). */
void oracle_channel_range(size_t count, size_t esize, int nchannels, int c,
                          size_t* lo, size_t* hi) {
  size_t a = 16 / esize;
  size_t per = align_up(div_up(count, (size_t)nchannels), a);
  *lo = min_sz(count, (size_t)c * per);
  *hi = min_sz(count, *lo + per);
}

/* Elements per chunk in the loop that starts at offset `off` of a channel of
 * length `len`: the configured chunk for full loops, else the last-loop rule. */
size_t oracle_loop_chunk(size_t len, size_t off, size_t esize, int nranks,
                         size_t chunk_elems) {
  size_t a = 16 / esize;
  size_t loop = (size_t)nranks * chunk_elems;
  size_t rem = len - off;
  return rem < loop ? align_up(div_up(rem, (size_t)nranks), a) : chunk_elems;
}

/* Chunk k of a loop with `rem` elements left and chunk size `cur`:
 * [k*cur, min(rem, (k+1)*cur)) relative to the loop start; may be empty. */
static void chunk_span(size_t rem, size_t cur, int k, size_t* start, size_t* len) {
  size_t s = (size_t)k * cur;
  if (s >= rem) { *start = rem; *len = 0; return; }
  *start = s;
  *len = min_sz(cur, rem - s);
}

/* Chunk id of every element, for tests that need each element's fold order. */
int oracle_element_chunks(size_t count, int dtype, int nranks, int nchannels,
                          size_t chunk_elems, int32_t* chunk_of) {
  size_t es = elem_size(dtype);
  if (!es || nranks < 1 || nchannels < 1 || chunk_elems == 0) return -1;
  if (chunk_elems % (16 / es)) return -1;
  for (int c = 0; c < nchannels; c++) {
    size_t lo, hi;
    oracle_channel_range(count, es, nchannels, c, &lo, &hi);
    size_t len = hi - lo;
    for (size_t off = 0; off < len; off += (size_t)nranks * chunk_elems) {
      size_t cur = oracle_loop_chunk(len, off, es, nranks, chunk_elems);
      for (int k = 0; k < nranks; k++) {
        size_t s, l;
        chunk_span(len - off, cur, k, &s, &l);
        for (size_t e = 0; e < l; e++) chunk_of[lo + off + s + e] = k;
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------
 * One loop of the ring schedule over all ring indices (step 4).
 * base: first element of the loop; rem: elements left in the channel from
 * base; cur: chunk size of this loop.  pay_old/pay_new: n payload buffers of
 * cur elements each (what every ring index last sent).
 * --------------------------------------------------------------------- */
static void ring_loop(int n, int dtype, int op, size_t es, const int* ring,
                      const void* const* x, void* const* y, size_t base,
                      size_t rem, size_t cur, unsigned char** pay_old,
                      unsigned char** pay_new) {
  for (int s = 0; s <= 2 * n - 2; s++) {
    for (int i = 0; i < n; i++) {
      int prev = (i + n - 1) % n;                  /* ring predecessor */
      int k = ((i + n - 1 - s) % n + n) % n;       /* chunk of this stage */
      size_t st, len;
      chunk_span(rem, cur, k, &st, &len);
      const unsigned char* mine = (const unsigned char*)x[ring[i]] + (base + st) * es;
      unsigned char* out = (unsigned char*)y[ring[i]] + (base + st) * es;
      if (s == 0) {
        /* send: own chunk straight into the successor's FIFO */
        memcpy(pay_new[i], mine, len * es);
      } else if (s <= n - 2) {
        /* recvReduceSend: reduce the received chunk with our own, forward */
        combine(dtype, hop_op(op), pay_old[prev], mine, pay_new[i], len);
      } else if (s == n - 1) {
        /* recvReduceCopySend: last reduction, the chunk is final (postOp):
         * keep it in our output and forward it */
        combine(dtype, hop_op(op), pay_old[prev], mine, pay_new[i], len);
        if (op == OR_AVG) average(dtype, pay_new[i], len, n);
        memcpy(out, pay_new[i], len * es);
      } else if (s <= 2 * n - 3) {
        /* recvCopySend: all-gather hop: keep the final chunk and forward */
        memcpy(pay_new[i], pay_old[prev], len * es);
        memcpy(out, pay_new[i], len * es);
      } else {
        /* recv: the last final chunk arrives; nothing is forwarded */
        memcpy(out, pay_old[prev], len * es);
      }
    }
    unsigned char** t = pay_old; pay_old = pay_new; pay_new = t;
  }
}

/*
 * Ring AllReduce over n virtual ranks, channels [c_begin, c_end) only.
 * Channels own disjoint element ranges and run independently of each other
 * ([ARCH] §九.3: one channel is one block on its own slice of the buffer), so
 * calls for disjoint channel ranges may run at the same time (the benchmark's
 * threaded timing does); together they compute exactly what one call over
 * every channel computes.
 *   x[r], y[r]: rank r's input and output (count elements each; may alias).
 *   ring[i]:    rank at ring index i (NULL = identity); i sends to i+1 mod n.
 *   chunk_elems: per-rank, per-channel chunk of a full loop, a multiple of
 *               16 bytes.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_ring_allreduce_channels(int nranks, size_t count, int dtype, int op,
                                   int nchannels, size_t chunk_elems, const int* ring,
                                   const void* const* x, void* const* y,
                                   int c_begin, int c_end) {
  size_t es = elem_size(dtype);
  if (!es || op < OR_SUM || op > OR_AVG || nranks < 1 || nchannels < 1) return -1;
  if (chunk_elems == 0 || chunk_elems % (16 / es)) return -1;
  if (c_begin < 0 || c_end > nchannels || c_begin > c_end) return -1;
  int* order = malloc(sizeof(int) * (size_t)nranks);
  if (!order) return -1;
  for (int i = 0; i < nranks; i++) order[i] = ring ? ring[i] : i;

  if (nranks == 1) {                   /* a single rank only copies */
    for (int c = c_begin; c < c_end; c++) {
      size_t lo, hi;
      oracle_channel_range(count, es, nchannels, c, &lo, &hi);
      if (x[order[0]] != y[order[0]] && hi > lo)
        memcpy((unsigned char*)y[order[0]] + lo * es, (const unsigned char*)x[order[0]] + lo * es,
               (hi - lo) * es);
    }
    free(order);
    return 0;
  }

  size_t maxcur = chunk_elems;
  unsigned char** pa = calloc((size_t)nranks, sizeof(void*));
  unsigned char** pb = calloc((size_t)nranks, sizeof(void*));
  int rc = 0;
  for (int i = 0; i < nranks && pa && pb; i++) {
    pa[i] = malloc(maxcur * es);
    pb[i] = malloc(maxcur * es);
    if (!pa[i] || !pb[i]) rc = -1;
  }
  if (!pa || !pb) rc = -1;

  for (int c = c_begin; c < c_end && rc == 0; c++) {
    size_t lo, hi;
    oracle_channel_range(count, es, nchannels, c, &lo, &hi);
    size_t len = hi - lo;
    for (size_t off = 0; off < len; off += (size_t)nranks * chunk_elems) {
      size_t cur = oracle_loop_chunk(len, off, es, nranks, chunk_elems);
      ring_loop(nranks, dtype, op, es, order, x, y, lo + off, len - off, cur, pa, pb);
    }
  }

  for (int i = 0; i < nranks; i++) {
    if (pa) free(pa[i]);
    if (pb) free(pb[i]);
  }
  free(pa);
  free(pb);
  free(order);
  return rc;
}

/* Ring AllReduce over every channel (arguments as above). */
int oracle_ring_allreduce(int nranks, size_t count, int dtype, int op,
                          int nchannels, size_t chunk_elems, const int* ring,
                          const void* const* x, void* const* y) {
  return oracle_ring_allreduce_channels(nranks, count, dtype, op, nchannels, chunk_elems, ring, x, y, 0,
                                        nchannels);
}

/* ---------------------------------------------------------------------
 * The two halves of the ring as calls of their own ([ARCH] §七.1: the ring
 * runs reduce_scatter and all_gather as n-1 steps each, runRing).  The pages
 * give no buffer layout for these calls; the plain one is taken: a
 * ReduceScatter input holds n blocks of `count` elements and rank r's output
 * is block r reduced over all ranks; an AllGather output holds n blocks and
 * block q is rank q's input.  Ring index i finishes the block of rank
 * ring[i], so each stage visits whole blocks: chunk k of a stage is the block
 * of rank ring[k].  Channels and loops only cut every block into the same
 * pieces and change no element's fold order, so each block runs as one
 * chunk here.
 * --------------------------------------------------------------------- */

static int* ring_order_copy(int n, const int* ring) {
  int* order = malloc(sizeof(int) * (size_t)n);
  if (order)
    for (int i = 0; i < n; i++) order[i] = ring ? ring[i] : i;
  return order;
}

static unsigned char** payloads(int n, size_t bytes) {
  unsigned char** p = calloc((size_t)n, sizeof(void*));
  if (!p) return NULL;
  for (int i = 0; i < n; i++)
    if (!(p[i] = malloc(bytes ? bytes : 1))) {
      for (int j = 0; j < i; j++) free(p[j]);
      free(p);
      return NULL;
    }
  return p;
}

static void free_payloads(int n, unsigned char** p) {
  if (!p) return;
  for (int i = 0; i < n; i++) free(p[i]);
  free(p);
}

/*
 * Ring ReduceScatter: x[r] holds n*count elements, y[r] count elements (y[r]
 * may be x[r]'s block r).  Per stage s = 0..n-1, ring index i visits chunk
 * (i + n - 1 - s) mod n: send at s = 0, recvReduceSend up to s = n-2, and at
 * s = n-1 (its own chunk) the last reduction goes to its output and is not
 * forwarded.  Returns 0, or -1 on bad arguments.
 */
int oracle_ring_reduce_scatter(int nranks, size_t count, int dtype, int op, const int* ring,
                               const void* const* x, void* const* y) {
  size_t es = elem_size(dtype);
  if (!es || op < OR_SUM || op > OR_AVG || nranks < 1) return -1;
  int n = nranks;
  int* order = ring_order_copy(n, ring);
  if (!order) return -1;
  if (n == 1) {
    memmove(y[order[0]], x[order[0]], count * es);
    free(order);
    return 0;
  }
  unsigned char** pa = payloads(n, count * es);
  unsigned char** pb = payloads(n, count * es);
  int rc = (pa && pb) ? 0 : -1;
  for (int s = 0; s <= n - 1 && rc == 0; s++) {
    for (int i = 0; i < n; i++) {
      int prev = (i + n - 1) % n;
      int k = ((i + n - 1 - s) % n + n) % n;
      const unsigned char* mine = (const unsigned char*)x[order[i]] + (size_t)order[k] * count * es;
      if (s == 0)
        memcpy(pb[i], mine, count * es);                       /* send */
      else if (s <= n - 2)
        combine(dtype, hop_op(op), pa[prev], mine, pb[i], count);      /* recvReduceSend */
      else {
        combine(dtype, hop_op(op), pa[prev], mine, y[order[i]], count); /* recvReduceCopy */
        if (op == OR_AVG) average(dtype, y[order[i]], count, n);        /* postOp */
      }
    }
    unsigned char** t = pa; pa = pb; pb = t;
  }
  free_payloads(n, pa);
  free_payloads(n, pb);
  free(order);
  return rc;
}

/*
 * Ring AllGather of `count` elements of `esize` bytes per rank: y[r] holds n
 * blocks (x[r] may be y[r]'s block r).  Per stage s = 0..n-1, ring index i
 * handles the block of rank ring[(i - s) mod n]: at s = 0 it copies its own
 * input to its output and sends it, then receives, keeps and forwards
 * (recvCopySend) up to s = n-2, and at s = n-1 only receives.
 */
int oracle_ring_all_gather(int nranks, size_t count, size_t esize, const int* ring,
                           const void* const* x, void* const* y) {
  if (nranks < 1 || esize == 0) return -1;
  int n = nranks;
  size_t bytes = count * esize;
  int* order = ring_order_copy(n, ring);
  if (!order) return -1;
  unsigned char** pa = payloads(n, bytes);
  unsigned char** pb = payloads(n, bytes);
  int rc = (pa && pb) ? 0 : -1;
  for (int s = 0; s <= n - 1 && rc == 0; s++) {
    for (int i = 0; i < n; i++) {
      int prev = (i + n - 1) % n;
      int k = ((i - s) % n + n) % n;
      unsigned char* out = (unsigned char*)y[order[i]] + (size_t)order[k] * bytes;
      if (s == 0) {
        memcpy(pb[i], x[order[i]], bytes);                     /* copySend */
        memmove(out, x[order[i]], bytes);
      } else if (s <= n - 2) {
        memcpy(pb[i], pa[prev], bytes);                        /* recvCopySend */
        memcpy(out, pa[prev], bytes);
      } else {
        memcpy(out, pa[prev], bytes);                          /* recv */
      }
    }
    unsigned char** t = pa; pa = pb; pb = t;
  }
  free_payloads(n, pa);
  free_payloads(n, pb);
  free(order);
  return rc;
}

/* ---------------------------------------------------------------------
 * Tree AllReduce over a double binary tree ([ARCH] §五.4 "double binary
 * tree", §九.1 and §九.4: Tree all_reduce first reduces up the tree to the
 * root, then the root broadcasts the result back down; [BOOK] ch. 4 of the
 * Japanese edition, ncclGetBtree / ncclGetDtree).  Every virtual rank is one
 * vertex of the tree (one rank per node, so there is no intra-node chain).
 *
 * Readings where the pages are silent:
 *   - the two trees each carry half of the data: channel c runs on tree
 *     c mod 2 (with one channel, tree 0 carries everything);
 *   - a vertex folds its own input first and then its children in child-slot
 *     order: acc = x; acc = op(P(child 0), acc); acc = op(P(child 1), acc),
 *     with op(received, local) as on the ring;
 *   - the odd-n second tree shifts every rank by one: it is the binary tree
 *     of rank (r - 1) mod n with every rank it names moved back by +1 mod n;
 *   - channels split the buffer as on the ring, and each channel's range is
 *     cut into chunks of chunk_elems elements (the last one shorter); a
 *     chunk goes all the way up and down before the next one.
 * --------------------------------------------------------------------- */

/*
 * Binary tree over ranks 0..n-1 (the pages' bit construction).  For a rank
 * r > 0 let b be its lowest set bit.  The parent clears b and sets the next
 * higher bit; if that is not a rank, it only clears b.  Children are r - b/2
 * (slot 0) and r + h (slot 1) for the largest h in b/2, b/4, ..., 1 with
 * r + h < n; a rank with b == 1 is a leaf.  Rank 0 is the root: its only
 * child (slot 1) is B/2, B the smallest power of two >= n.  -1 = none.
 */
void oracle_btree(int n, int r, int* up, int* down0, int* down1) {
  int b = 1;
  while (b < n && (r & b) == 0) b <<= 1;   /* r's lowest set bit (r = 0: B) */
  if (r == 0) {
    *up = -1;
    *down0 = -1;
    *down1 = n > 1 ? b / 2 : -1;
    return;
  }
  int parent = (r & ~b) | (b << 1);
  if (parent >= n) parent = r & ~b;
  *up = parent;
  int h = b / 2;
  *down0 = h > 0 ? r - h : -1;
  while (h > 0 && r + h >= n) h /= 2;
  *down1 = h > 0 ? r + h : -1;
}

/* Tree t (0 or 1) of the double binary tree: tree 0 is the binary tree;
 * tree 1 is its mirror image (rank r plays rank n-1-r) when n is even, and
 * the binary tree shifted by one rank when n is odd. */
void oracle_dtree(int n, int r, int t, int* up, int* down0, int* down1) {
  if (t == 0) {
    oracle_btree(n, r, up, down0, down1);
    return;
  }
  int u, d0, d1;
  if (n % 2 == 0) {
    oracle_btree(n, n - 1 - r, &u, &d0, &d1);
    *up = u < 0 ? -1 : n - 1 - u;
    *down0 = d0 < 0 ? -1 : n - 1 - d0;
    *down1 = d1 < 0 ? -1 : n - 1 - d1;
  } else {
    oracle_btree(n, (r - 1 + n) % n, &u, &d0, &d1);
    *up = u < 0 ? -1 : (u + 1) % n;
    *down0 = d0 < 0 ? -1 : (d0 + 1) % n;
    *down1 = d1 < 0 ? -1 : (d1 + 1) % n;
  }
}

/*
 * Tree AllReduce of n virtual ranks (x[r], y[r]: count elements each; they
 * may alias for the in-place form).  Per channel, per chunk: the reduce
 * phase visits vertices deepest first, so every child's partial result P
 * exists before its parent folds it in; the root's P is the result; the
 * broadcast phase then visits vertices shallowest first, each taking the
 * result from its parent and storing it in its output.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_tree_allreduce(int nranks, size_t count, int dtype, int op, int nchannels,
                          size_t chunk_elems, const void* const* x, void* const* y) {
  size_t es = elem_size(dtype);
  int n = nranks;
  if (!es || op < OR_SUM || op > OR_AVG || n < 1 || nchannels < 1 || chunk_elems == 0) return -1;
  if (n == 1) {
    memmove(y[0], x[0], count * es);
    return 0;
  }
  int* up = malloc(sizeof(int) * (size_t)n);
  int* dn = malloc(sizeof(int) * 2 * (size_t)n);
  int* depth = malloc(sizeof(int) * (size_t)n);
  int* order = malloc(sizeof(int) * (size_t)n);   /* vertices, deepest first */
  unsigned char** P = payloads(n, chunk_elems * es);
  int rc = (up && dn && depth && order && P) ? 0 : -1;
  for (int c = 0; c < nchannels && rc == 0; c++) {
    int t = c % 2, root = -1;
    for (int r = 0; r < n; r++) {
      oracle_dtree(n, r, t, &up[r], &dn[2 * r], &dn[2 * r + 1]);
      if (up[r] < 0) root = r;
    }
    for (int r = 0; r < n; r++) {
      depth[r] = 0;
      for (int v = r; up[v] >= 0 && depth[r] <= n; v = up[v]) depth[r]++;
    }
    int k = 0;
    for (int d = n; d >= 0; d--)
      for (int r = 0; r < n; r++)
        if (depth[r] == d) order[k++] = r;
    if (root < 0 || k != n) { rc = -1; break; }

    size_t lo, hi;
    oracle_channel_range(count, es, nchannels, c, &lo, &hi);
    for (size_t off = lo; off < hi; off += chunk_elems) {
      size_t len = min_sz(chunk_elems, hi - off);
      /* reduce: up the tree */
      for (int j = 0; j < n; j++) {
        int v = order[j];
        memcpy(P[v], (const unsigned char*)x[v] + off * es, len * es);
        for (int s = 0; s < 2; s++) {
          int ch = dn[2 * v + s];
          if (ch >= 0) combine(dtype, hop_op(op), P[ch], P[v], P[v], len);
        }
        if (v == root && op == OR_AVG) average(dtype, P[v], len, n);   /* final: postOp */
      }
      /* broadcast: down the tree */
      for (int j = n - 1; j >= 0; j--) {
        int v = order[j];
        if (v != root) memcpy(P[v], P[up[v]], len * es);
        memcpy((unsigned char*)y[v] + off * es, P[v], len * es);
      }
    }
  }
  free(up);
  free(dn);
  free(depth);
  free(order);
  free_payloads(n, P);
  return rc;
}

/* Array forms of the 16-bit codecs, for the tests' exhaustive pins. */
void oracle_f16_decode_array(const uint16_t* h, float* f, size_t len) {
  for (size_t e = 0; e < len; e++) f[e] = f16_decode(h[e]);
}
void oracle_f16_encode_array(const float* f, uint16_t* h, size_t len) {
  for (size_t e = 0; e < len; e++) h[e] = f16_encode_rne(f[e]);
}
void oracle_bf16_decode_array(const uint16_t* h, float* f, size_t len) {
  for (size_t e = 0; e < len; e++) f[e] = bf16_decode(h[e]);
}
void oracle_bf16_encode_array(const float* f, uint16_t* h, size_t len) {
  for (size_t e = 0; e < len; e++) h[e] = bf16_encode_rne(f[e]);
}
