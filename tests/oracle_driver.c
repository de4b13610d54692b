/*
 * Test driver for the CPU oracle (test infrastructure): runs the oracle's
 * collectives over cases read from a file and writes their outputs to
 * another, so that a build of oracle/ring_oracle.c with the address and
 * undefined-behaviour sanitizers can be driven by the Python brute-force
 * battery (tests/test_oracle_sanitized.py).  Every buffer is allocated at
 * its exact size, so any access past it is reported by the sanitizer.
 *
 * Case record (little-endian): int32 kind (0 ring AllReduce, 1 ReduceScatter,
 * 2 AllGather, 3 tree AllReduce), nranks, dtype, op, nchannels, in_place,
 * has_ring; uint64 count, chunk_elems; int32 ring[nranks] if has_ring; then
 * each rank's input.  Output: each rank's output, case after case.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_ring_allreduce(int, size_t, int, int, int, size_t, const int*, const void* const*, void* const*);
int oracle_ring_reduce_scatter(int, size_t, int, int, const int*, const void* const*, void* const*);
int oracle_ring_all_gather(int, size_t, size_t, const int*, const void* const*, void* const*);
int oracle_tree_allreduce(int, size_t, int, int, int, size_t, const void* const*, void* const*);

static const size_t kElem[6] = {1, 4, 2, 2, 4, 8};

static int read_all(FILE* f, void* p, size_t n) { return n == 0 || fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* in = fopen(argv[1], "rb");
  FILE* out = fopen(argv[2], "wb");
  if (!in || !out) return 2;
  int32_t h[7];
  int cases = 0;
  while (fread(h, sizeof(h), 1, in) == 1) {
    const int kind = h[0], n = h[1], dtype = h[2], op = h[3], nch = h[4], inplace = h[5], has_ring = h[6];
    uint64_t cc[2];
    if (!read_all(in, cc, sizeof(cc)) || n < 1 || n > 64 || dtype < 0 || dtype > 5) return 3;
    const size_t count = (size_t)cc[0], chunk = (size_t)cc[1], es = kElem[dtype];
    int* ring = NULL;
    if (has_ring) {
      ring = malloc(sizeof(int) * (size_t)n);
      int32_t* r32 = malloc(sizeof(int32_t) * (size_t)n);
      if (!ring || !r32 || !read_all(in, r32, sizeof(int32_t) * (size_t)n)) return 3;
      for (int i = 0; i < n; i++) ring[i] = r32[i];
      free(r32);
    }
    const size_t in_elems = kind == 1 ? (size_t)n * count : count;
    const size_t out_elems = kind == 2 ? (size_t)n * count : count;
    void** x = calloc((size_t)n, sizeof(void*));
    void** y = calloc((size_t)n, sizeof(void*));
    void** big = calloc((size_t)n, sizeof(void*));   /* the buffer that holds both, in place */
    if (!x || !y || !big) return 3;
    for (int r = 0; r < n; r++) {
      /* malloc(0) may return NULL; one byte keeps every pointer valid */
      const size_t ib = in_elems * es, ob = out_elems * es;
      if (!inplace) {
        x[r] = malloc(ib ? ib : 1);
        y[r] = malloc(ob ? ob : 1);
        if (!x[r] || !y[r] || !read_all(in, x[r], ib)) return 3;
        memset(y[r], 0xA5, ob);
      } else if (kind == 0 || kind == 3) {
        big[r] = malloc(ib ? ib : 1);
        if (!big[r] || !read_all(in, big[r], ib)) return 3;
        x[r] = y[r] = big[r];
      } else if (kind == 1) {   /* ReduceScatter: the output is the rank's own block of its input */
        big[r] = malloc(ib ? ib : 1);
        if (!big[r] || !read_all(in, big[r], ib)) return 3;
        x[r] = big[r];
        y[r] = (char*)big[r] + (size_t)r * count * es;
      } else {                  /* AllGather: the input is the rank's own block of its output */
        big[r] = malloc(ob ? ob : 1);
        if (!big[r]) return 3;
        memset(big[r], 0xA5, ob);
        y[r] = big[r];
        x[r] = (char*)big[r] + (size_t)r * count * es;
        if (!read_all(in, x[r], ib)) return 3;
      }
    }
    int rc;
    if (kind == 0) rc = oracle_ring_allreduce(n, count, dtype, op, nch, chunk, ring, (const void* const*)x, y);
    else if (kind == 1) rc = oracle_ring_reduce_scatter(n, count, dtype, op, ring, (const void* const*)x, y);
    else if (kind == 2) rc = oracle_ring_all_gather(n, count, es, ring, (const void* const*)x, y);
    else rc = oracle_tree_allreduce(n, count, dtype, op, nch, chunk, (const void* const*)x, y);
    if (rc != 0) return 4;
    for (int r = 0; r < n; r++)
      if (out_elems && fwrite(y[r], es, out_elems, out) != out_elems) return 5;
    for (int r = 0; r < n; r++) {
      if (inplace) free(big[r]);
      else { free(x[r]); free(y[r]); }
    }
    free(x); free(y); free(big); free(ring);
    cases++;
  }
  fclose(in);
  fclose(out);
  printf("%d cases\n", cases);
  return 0;
}
