/*
 * ringar: ring AllReduce (and its two halves, ReduceScatter and AllGather)
 * over n virtual ranks that all live in one MI355X, and the tree AllReduce
 * over the pages' double binary tree.
 *
 * The operation is the device-side ring AllReduce described on
 *   [ARCH] arganzheng.life, "NCCL architecture: topology, channels, algorithms
 *          and protocols": §九.4 (runRing: send, recvReduceSend x (n-2),
 *          recvReduceCopySend, recvCopySend x (n-2), recv), §七.2 (the Simple,
 *          LL and LL128 protocols), §六.5 (a FIFO of 8 steps per connection),
 *          §八 (the alpha-beta tuning model), §九.1 (argument checks).
 *   [BOOK] aireadcode.com, "NCCL Source Code Deep Dive: A GPU Journey of One
 *          AllReduce": §1.3 (ncclAllReduce(sendbuff, recvbuff, count,
 *          datatype, op, comm, stream) only enqueues; results are valid after
 *          a stream synchronisation), §2.3 (chunk id and last-loop chunk size),
 *          ch. 6 of the Japanese edition (count == 0 is a no-op; one rank is a
 *          local copy; error classes).
 *
 * Every rank r contributes sendbuffs[r] (count elements) and receives in
 * recvbuffs[r] the elementwise reduction over all ranks, identical on every
 * rank.  All buffers, FIFO slots and step counters are in one GPU's HBM; a
 * "rank" is a set of workgroups of one kernel launch.
 *
 * Threading: calls are host-thread safe.  Calls on one stream run in stream
 * order and share that stream's FIFO memory; calls on different streams use
 * different FIFO memory and may run concurrently if the GPU has room for both
 * grids.
 *
 * Co-residency: every wavefront of a launch waits on others of the same
 * launch, so the whole grid must be resident at once.  The library checks its
 * own grid against what the GPU holds of that kernel, but it cannot see other
 * work: a call that overlaps another large kernel (another ringar call on a
 * second stream, or another process's kernels) may find part of its grid
 * unscheduled until that work ends.  Its waits then run into the spin limit
 * and the call reports RINGAR_ERR_TIMEOUT through ringar_get_async_error
 * (bounded, never a hang).  Do not overlap large calls with other large
 * kernels on the same GPU.
 */
#ifndef RINGAR_H
#define RINGAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (declared here so the header needs no HIP headers).
 * NULL is the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t* ringar_stream_t;

typedef enum {
  RINGAR_SUCCESS = 0,
  RINGAR_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, enum, ring order, ... */
  RINGAR_ERR_INVALID_USAGE = 2,    /* a valid request this GPU/config cannot run */
  RINGAR_ERR_INTERNAL = 3,
  RINGAR_ERR_DEVICE = 4,           /* a HIP call failed; see ringar_last_error() */
  RINGAR_ERR_ABORTED = 5,          /* the abort word was set while the kernel waited */
  RINGAR_ERR_TIMEOUT = 6           /* a wait exceeded the spin limit */
} ringar_result_t;

typedef enum {
  RINGAR_INT8 = 0,
  RINGAR_INT32 = 1,
  RINGAR_FLOAT16 = 2,
  RINGAR_BFLOAT16 = 3,
  RINGAR_FLOAT32 = 4,
  RINGAR_FLOAT64 = 5
} ringar_dtype_t;

/* sum and prod wrap for integers; fp16/bf16 apply the op in fp32 and round to
 * nearest-even on every hop; min/max keep the received value on ties.
 * avg folds every hop like sum and divides each final value by nranks once,
 * at the step where it becomes final (the postOp of [ARCH] §九.4's
 * recvReduceCopySend; for the tree, at the root): integers truncate toward
 * zero, fp32/fp64 divide once, fp16/bf16 divide in fp32 and round to
 * nearest-even. */
typedef enum { RINGAR_SUM = 0, RINGAR_PROD = 1, RINGAR_MIN = 2, RINGAR_MAX = 3, RINGAR_AVG = 4 } ringar_op_t;

/* Protocol codes follow the pages' protocol table order {LL, LL128, Simple}.
 *   LL:     8-byte FIFO lines, 4 B data + 4 B flag, one 64-bit store each.
 *   LL128:  128-byte FIFO lines, 120 B data + 8 B flag.
 *   Simple: plain FIFO slots plus a tail counter (producer) and a head
 *           counter (consumer), 8 slots per connection. */
typedef enum {
  RINGAR_PROTO_AUTO = -1,
  RINGAR_PROTO_LL = 0,
  RINGAR_PROTO_LL128 = 1,
  RINGAR_PROTO_SIMPLE = 2
} ringar_proto_t;

/* Collectives of ringar_plan_coll: the AllReduce and its two halves, which
 * the ring also runs as calls of their own ([ARCH] §七.1: reduce_scatter and
 * all_gather take n-1 ring steps each). */
typedef enum {
  RINGAR_ALLREDUCE = 0,
  RINGAR_REDUCE_SCATTER = 1,
  RINGAR_ALL_GATHER = 2
} ringar_coll_t;

/* AllReduce algorithms ([ARCH] §七.1: Ring, and Tree = reduce up a double
 * binary tree to its root, then broadcast back down; the tuning model runs
 * Tree for AllReduce only).
 *   RING: the ring of the pages' runRing (the default: 0 in a zeroed config).
 *   TREE: the double binary tree of [ARCH] §五.4 over the n virtual ranks,
 *         each rank one tree vertex; channel c runs on tree c % 2.  A vertex
 *         folds its own input, then child 0's and child 1's partial results,
 *         each hop as op(received, local); every rank receives the root's
 *         result.
 *   AUTO: the model's fastest (algorithm, protocol) pair among those the
 *         environment allows (RINGAR_ALGO: "ring", "tree", a list, or '^' to
 *         exclude, like RINGAR_PROTO). */
typedef enum {
  RINGAR_ALGO_RING = 0,
  RINGAR_ALGO_TREE = 1,
  RINGAR_ALGO_AUTO = 2
} ringar_algo_t;

/* Inputs of the alpha-beta model ([ARCH] §八.1-八.2), per protocol in the
 * order LL, LL128, Simple.  Bandwidths GB/s, latencies microseconds.
 *   bus bandwidth:  nch * bw_per_channel * eff[p], LL capped at ll_max_bw,
 *                   LL128 capped at nch * ll128_per_channel_max_bw;
 *   alg bandwidth:  bus * n / (2(n-1));
 *   latency:        base_lat_us[p] + 2(n-1) * hw_lat_us[p];
 *   time:           latency + bytes / (1000 * alg bandwidth).
 * Channel auto rule ([ARCH] §六.4): start at min(max_channels,
 * max_pairs / n) and drop one channel while
 * bytes < nch * threads[p] * thread_threshold[p] (LL: times n). */
typedef struct {
  double bw_per_channel;
  double ll_max_bw;
  double ll128_per_channel_max_bw;
  double eff[3];
  double base_lat_us[3];
  double hw_lat_us[3];
  int max_channels;
  int max_pairs;
  int threads[3];
  int thread_threshold[3];
  size_t default_chunk_bytes[3];
  /* Tree rows ([BOOK] Japanese edition ch. 5 §四; [ARCH] §八.1), with every
   * virtual rank one tree vertex (one rank per node):
   *   bus bandwidth: min(nch * bw_per_channel * tree_allreduce_eff,
   *                      nch * tree_per_channel_max_bw);
   *                  LL: that / tree_ll_divisor, capped at ll_max_bw;
   *                  LL128: that * tree_ll128_factor, capped at
   *                  nch * tree_ll128_per_channel_max_bw;
   *   alg bandwidth: bus * 0.5, times the pages' size correction table when
   *                  tree_correction is 1;
   *   latency:       tree_base_lat_us[p] + 2 * floor(log2 n) * tree_hw_lat_us[p]. */
  double tree_allreduce_eff;
  double tree_per_channel_max_bw;
  double tree_ll_divisor;
  double tree_ll128_factor;
  double tree_ll128_per_channel_max_bw;
  double tree_base_lat_us[3];
  double tree_hw_lat_us[3];
  int tree_correction;
} ringar_model_t;

/* Optional knobs of ringar_allreduce_ex.  Zero-initialise, then set fields.
 *   chunk_bytes:     per-rank, per-channel chunk of one ring step; a multiple
 *                    of 16 bytes; 0 = the protocol's default.
 *   ring_order:      host array of nranks ints: rank at ring index i (ring
 *                    index i sends to i+1 mod n); NULL = identity.  Must be a
 *                    permutation of 0..n-1.
 *   model:           model for AUTO choices; NULL = built-in MI355X model.
 *   lanes:           wavefronts working in parallel on each (rank, channel),
 *                    each with its own FIFO; 0 = chosen by size (a power of
 *                    two, or a multiple of 4 when that saves a FIFO slice).
 *                    A forced count must be a power of two, at most 32;
 *                    one whose grid the GPU cannot hold at once is refused
 *                    with RINGAR_ERR_INVALID_USAGE (by ringar_plan too when
 *                    a device is visible).  Does not change any result.
 *   spin_limit_ms:   a wait that lasts longer ends the kernel with
 *                    RINGAR_ERR_TIMEOUT (reported by ringar_get_async_error);
 *                    0 = default (env RINGAR_SPIN_LIMIT_MS, else 2000 ms).
 *   abort_flag:      host-mapped (pinned) word, or NULL.  While nonzero, any
 *                    waiting wavefront gives up with RINGAR_ERR_ABORTED.
 *   skip_rank:       test hook, normally -1: every wavefront of this rank
 *                    returns at once, so its peers must time out or abort.
 *   fifo_depth:      FIFO slots each connection cycles through: 2, 4 or 8
 *                    (the pages' NCCL_STEPS is 8); 0 = chosen by size.  A
 *                    lane's part of a chunk may fill at most half of them,
 *                    else RINGAR_ERR_INVALID_USAGE.  Does not change any
 *                    result.
 *   force_general:   test hook, normally 0: 1 = never use the straight-line
 *                    form for small lane parts (see ringar_plan_t).
 *   algo:            a ringar_algo_t (AllReduce only; the halves run the
 *                    ring).  Zero = RINGAR_ALGO_RING.
 *   direct:          the direct form: the ring AllReduce under Simple
 *                    writes each outgoing slice straight into the
 *                    successor's receive buffer instead of a FIFO slot (the
 *                    pages' direct primitives, [ARCH] §九.4): fewer bytes
 *                    moved, same results.  1 = whenever the call is a ring
 *                    AllReduce with the Simple protocol (a captured call is
 *                    then refused); 2 = never; 0 = the library's choice:
 *                    when proto is RINGAR_PROTO_AUTO and the model takes
 *                    Simple on the ring for at least 256 KiB per rank
 *                    (outside stream capture).  It needs every rank out of
 *                    place; otherwise the call runs with FIFOs as usual.
 *   block_map:       which workgroup runs which (rank, channel, lane): 0 =
 *                    by size (the XCD-major mapping up to 512 KiB per rank,
 *                    LL128 up to 32 KiB, else linear; linear too where the
 *                    XCD-major grid, padded to whole rounds of 8 groups,
 *                    would not be resident at once), 1 = linear, 2 =
 *                    XCD-major (every rank of a channel on one of MI355X's
 *                    8 XCDs; RINGAR_ERR_INVALID_USAGE where its padded grid
 *                    is not resident at once).  Changes speed only, never
 *                    a result. */
typedef struct {
  size_t chunk_bytes;
  const int* ring_order;
  const ringar_model_t* model;
  int lanes;
  uint32_t spin_limit_ms;
  volatile uint32_t* abort_flag;
  int skip_rank;
  int fifo_depth;
  int force_general;
  int algo;
  int direct;
  int block_map;
} ringar_config_t;

/* The resolved plan of a call (what ringar_allreduce would launch). */
typedef struct {
  ringar_proto_t proto;
  int nchannels;
  size_t chunk_bytes;
  size_t chunk_elems;
  size_t align_elems;      /* 16 B / element size */
  size_t channel_elems;    /* per-channel length before clipping to count */
  int lanes;               /* wavefronts per (rank, channel) */
  int fifo_depth;          /* FIFO slots in use per connection */
  int small_slices;        /* 1: every lane part is at most 1 KiB, and LL or
                              Simple run their straight-line form (one 16-byte
                              packet per lane and step) when all buffers are
                              16-byte aligned */
  int workgroups;          /* grid size */
  int threads_per_group;
  uint64_t max_steps;      /* upper bound on FIFO steps per connection */
  double predicted_us[3];  /* model time per protocol (LL, LL128, Simple) of
                              the plan's algorithm */
  ringar_algo_t algo;      /* RING or TREE */
  double predicted_tree_us[3];  /* Tree AllReduce model times (AllReduce) */
  double predicted_ring_us[3];  /* Ring model times */
  int direct;              /* 1: runs the direct form when every rank is out
                              of place */
  int xcd_major;           /* 1: XCD-major block mapping (see block_map) */
  int tree_split;          /* 1: the tree's split form: each role that moves
                              four or more units per element runs as two
                              wavefronts on halves of every slice */
  int tree_waves_per_lane; /* the split form's wavefronts per (channel,
                              lane); 0 otherwise */
} ringar_plan_t;

/*
 * Ring AllReduce of n = nranks virtual ranks ([BOOK] §1.3 signature with a
 * communicator replaced by the rank count).
 *   sendbuffs, recvbuffs: host arrays of nranks DEVICE pointers; rank r reads
 *       count elements at sendbuffs[r] and writes count elements at
 *       recvbuffs[r].  sendbuffs[r] == recvbuffs[r] (in place) is allowed;
 *       any other overlap between the 2n buffers is RINGAR_ERR_INVALID_USAGE.
 *       Pointers must be aligned to the element size; 16-byte aligned
 *       pointers take the vector path.  The caller owns all buffers; the
 *       host arrays are read only during the call.
 *   count: elements per rank.  0 is a successful no-op.
 *   nchannels: 1..64, or 0 = chosen by the model's size rule.
 *   proto: a protocol, or RINGAR_PROTO_AUTO = the model's fastest (where it
 *       is Simple from 256 KiB per rank, out of place and outside stream
 *       capture, the call runs the direct form; see ringar_config_t).
 *   stream: the work is enqueued on this stream; results are valid after the
 *       stream has been synchronised.  nranks == 1 enqueues a device copy.
 *       Under stream capture (a HIP graph, replayed any number of times)
 *       every collective here (AllReduce by ring or tree, ReduceScatter,
 *       AllGather) runs a captured form: its steps count from zero on
 *       counters of its own and it leaves every counter and flag it
 *       consumed at zero, so each replay starts clean and eager calls on
 *       the stream keep working between replays.  Nothing is allocated or
 *       cleared during capture: the stream must have run a call of the same
 *       shape first (else RINGAR_ERR_INVALID_USAGE).  The captured kernels
 *       may hold fewer wavefronts per CU, so a captured call can take fewer
 *       lanes than the same call made eagerly (same results); a forced lane
 *       count beyond what they hold is RINGAR_ERR_INVALID_USAGE.  The tree
 *       never runs its split form under capture (it may then take more
 *       lanes and another chunk, same results); an eager call in the split
 *       form allocates the connections of both forms.  A call that
 *       asks for the direct form is refused under capture
 *       (RINGAR_ERR_INVALID_USAGE, nothing enqueued); one for which the
 *       library chose it keeps its FIFOs.
 *       Replays share the stream's FIFO memory with its eager calls: run
 *       them in order (one stream, or synchronised).  A graph holds the
 *       addresses of the stream's FIFO memory and counters: later eager
 *       calls that need more of them keep the old buffers alive for it, and
 *       ringar_release frees them, so a graph captured before
 *       ringar_release must not be replayed after it.  After an
 *       asynchronous error in a replay, call ringar_get_async_error (it
 *       resets what the failed replay left behind) before replaying again.
 * Errors are reported before anything is enqueued; a wait that times out or
 * is aborted inside the kernel is reported by ringar_get_async_error.
 */
ringar_result_t ringar_allreduce(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                 ringar_dtype_t dtype, ringar_op_t op, int nranks,
                                 int nchannels, ringar_proto_t proto, ringar_stream_t stream);

/* As ringar_allreduce with the optional knobs of ringar_config_t (cfg may be
 * NULL). */
ringar_result_t ringar_allreduce_ex(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                    ringar_dtype_t dtype, ringar_op_t op, int nranks,
                                    int nchannels, ringar_proto_t proto, ringar_stream_t stream,
                                    const ringar_config_t* cfg);
/* With cfg->algo = RINGAR_ALGO_TREE (or AUTO choosing it) the same call runs
 * the tree AllReduce: buffers, in place, alignment, streams, errors, count ==
 * 0 and nranks == 1 as above.  The chunk is per channel (the tree moves a
 * whole chunk up and down, not one chunk per rank as the ring's loop), and
 * float results follow the tree's fold order, not the ring's. */

/*
 * The same AllReduce as ringar_allreduce_ex, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * hipMalloc): this entry point calls no hipMalloc, hipFree or other
 * allocating routine.  Its FIFO slots, counters and error word live in one
 * fixed device array of the library (64 MiB of FIFO slots, counters for 4096
 * connections, an error word; each GPU the library runs on holds its own copy
 * from the library's first use of that GPU until the process ends).  The
 * caller passes inputs and outputs as for ringar_allreduce_ex, with the same
 * meaning, checks and results: every choice that decides a result (protocol,
 * channels, chunk, algorithm, ring order) is the one ringar_plan reports; the
 * plan may take fewer lanes so that its connections fit the array (lanes
 * change no result).  A call whose connections do not fit even with one lane
 * per (rank, channel) (about 2 x nranks x nchannels x chunk bytes of FIFO),
 * or whose forced lane count does not fit, is refused with
 * RINGAR_ERR_INVALID_USAGE before anything is enqueued, the reason in
 * ringar_last_error().  Refused under stream capture (no captured form).
 * Every call on a GPU shares that GPU's array, which keeps what the last
 * call left: calls that overlap on one GPU (on different streams, or with
 * another thread's calls) race and must be avoided; calls in stream order,
 * or synchronised, are safe.  Asynchronous errors are reported by
 * ringar_get_async_error (synchronise the call's stream first).
 * ringar_release does not touch the array.
 */
ringar_result_t ringar_allreduce_noalloc(void* const* sendbuffs, void* const* recvbuffs, size_t count,
                                         ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                         ringar_proto_t proto, ringar_stream_t stream,
                                         const ringar_config_t* cfg);

/*
 * Ring ReduceScatter, the first half of the ring AllReduce as a call of its
 * own ([ARCH] §七.1; the pages give no buffer layout, the plain one is
 * taken): sendbuffs[r] holds nranks blocks of recvcount elements, and
 * recvbuffs[r] receives block r reduced over all ranks.  Ring index i
 * finishes the block of rank ring_order[i]; float results follow that ring's
 * fold order (the block starts at ring index i+1 and ring index i folds in
 * last).  In place: recvbuffs[r] == sendbuffs[r] + r * recvcount elements;
 * any other overlap with a receive buffer is RINGAR_ERR_INVALID_USAGE.
 * Alignment, streams, errors, nranks == 1 and count == 0 as in
 * ringar_allreduce; the vector path also needs recvcount * element size to
 * be a multiple of 16 bytes.
 */
ringar_result_t ringar_reduce_scatter(void* const* sendbuffs, void* const* recvbuffs, size_t recvcount,
                                      ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                      ringar_proto_t proto, ringar_stream_t stream);
ringar_result_t ringar_reduce_scatter_ex(void* const* sendbuffs, void* const* recvbuffs, size_t recvcount,
                                         ringar_dtype_t dtype, ringar_op_t op, int nranks, int nchannels,
                                         ringar_proto_t proto, ringar_stream_t stream,
                                         const ringar_config_t* cfg);

/*
 * Ring AllGather, the second half as a call of its own ([ARCH] §七.1; plain
 * layout): sendbuffs[r] holds sendcount elements, and every recvbuffs[q]
 * receives nranks blocks of sendcount elements, block r being rank r's
 * input, bit for bit (a byte copy: the dtype only sets the element size).
 * In place: sendbuffs[r] == recvbuffs[r] + r * sendcount elements.
 * Otherwise as ringar_reduce_scatter.
 */
ringar_result_t ringar_all_gather(void* const* sendbuffs, void* const* recvbuffs, size_t sendcount,
                                  ringar_dtype_t dtype, int nranks, int nchannels, ringar_proto_t proto,
                                  ringar_stream_t stream);
ringar_result_t ringar_all_gather_ex(void* const* sendbuffs, void* const* recvbuffs, size_t sendcount,
                                     ringar_dtype_t dtype, int nranks, int nchannels, ringar_proto_t proto,
                                     ringar_stream_t stream, const ringar_config_t* cfg);

/* Host only, no GPU needed: the plan ringar_allreduce_ex would use for these
 * arguments (cfg may be NULL).  Returns the same argument errors.
 *   The partition follows the pages: channels own contiguous ranges of the
 *   buffer ([BOOK] §2.2), a loop covers nranks chunks of chunk_elems and the
 *   last loop's chunks are alignUp(ceil(rem / nranks), 16 B / element size)
 *   elements ([BOOK] §2.3, RingARAlgorithm::getNextSendAddr); with
 *   nchannels == 0 the channel count comes from the size rule of [ARCH] §六.4
 *   (drop a channel while bytes < nch x threads x threshold), and with
 *   proto == RINGAR_PROTO_AUTO the protocol from the alpha-beta model of
 *   [ARCH] §八.1-八.2.  lanes, fifo_depth and small_slices are this
 *   library's own (they change no result).
 *   out: caller-owned, filled on success, untouched on error. */
ringar_result_t ringar_plan(size_t count, ringar_dtype_t dtype, int nranks, int nchannels,
                            ringar_proto_t proto, const ringar_config_t* cfg, ringar_plan_t* out);

/* Host only: the plan of any of the three collectives; count as in its call
 * (elements per rank, or per block for the halves).  The halves' model takes
 * n-1 ring steps and counts all n blocks as the call's size (the pages'
 * tuning rule for AllGather / ReduceScatter); their channel split applies to
 * one block, and a loop takes up to one chunk of every block.  AllGather
 * plans a byte copy: its chunk_elems, align_elems and channel_elems count
 * bytes. */
ringar_result_t ringar_plan_coll(ringar_coll_t coll, size_t count, ringar_dtype_t dtype, int nranks,
                                 int nchannels, ringar_proto_t proto, const ringar_config_t* cfg,
                                 ringar_plan_t* out);

/* Host only: the model's fastest protocol for `bytes` per rank over nchannels
 * channels (model NULL = built-in), ties going to Simple, then LL128
 * ([BOOK] ch. 5 of the Japanese edition: the first strictly smaller time in a
 * front-pushed candidate list wins).  predicted_us (may be NULL) receives the
 * three times. */
ringar_result_t ringar_select(size_t bytes, int nranks, int nchannels, const ringar_model_t* model,
                              ringar_proto_t* out, double* predicted_us);

/* Host only: the model's fastest (algorithm, protocol) pair for an
 * AllReduce of `bytes` per rank over nchannels channels (0 = the model's
 * maximum), among the pairs RINGAR_ALGO and RINGAR_PROTO allow.  The
 * candidates are numbered Tree LL, Tree LL128, Tree Simple, Ring LL, Ring
 * LL128, Ring Simple (the pages' model map) and visited in reverse, the
 * first strictly smaller time winning, so ties go to Ring Simple first.
 * predicted_us (may be NULL) receives the six times in that order. */
ringar_result_t ringar_select_algo(size_t bytes, int nranks, int nchannels, const ringar_model_t* model,
                                   ringar_algo_t* algo, ringar_proto_t* proto, double* predicted_us);

/* Host only: vertex `rank` of tree `tree` (0 or 1) of the double binary tree
 * the tree AllReduce uses over nranks ranks ([ARCH] §五.4): its parent and
 * its children in child-slot order, -1 = none. */
ringar_result_t ringar_tree(int nranks, int tree, int rank, int* parent, int* child0, int* child1);

/* Host only: the built-in MI355X model constants, in the form of the pages'
 * tuning model ([ARCH] §八.1-八.2; the pages' own constants are NVIDIA's);
 * the values are fitted to this library's calls on MI355X, which no page
 * gives.  out: caller-owned; RINGAR_ERR_INVALID_ARGUMENT if NULL. */
ringar_result_t ringar_default_model(ringar_model_t* out);

/* Host only: element range [lo, hi) of channel c and, for the loop starting
 * at element `loop_off` of that channel, chunk k's range [klo, khi)
 * (absolute element indices; empty ranges have klo == khi): the channel
 * split of [BOOK] §2.2 and the chunk rule of [BOOK] §2.3
 * (RingARAlgorithm::getNextSendAddr), as the kernels use them.  chunk_elems
 * must be a multiple of 16 bytes; every output pointer must be non-NULL,
 * else RINGAR_ERR_INVALID_ARGUMENT. */
ringar_result_t ringar_chunk_range(size_t count, ringar_dtype_t dtype, int nranks, int nchannels,
                                   size_t chunk_elems, int c, size_t loop_off, int k,
                                   size_t* lo, size_t* hi, size_t* klo, size_t* khi);

/* Asynchronous errors ([BOOK] §1.4: ncclCommGetAsyncError reports what went
 * wrong after the call returned; [ARCH] §九.5: a kernel only leaves its wait
 * loops through the abort flag).  Waits for `stream`, then returns (and
 * clears) the first error a kernel enqueued on this stream recorded:
 * RINGAR_ERR_TIMEOUT (a wait passed the spin limit), RINGAR_ERR_ABORTED (the
 * abort word was set), RINGAR_ERR_INTERNAL (a part larger than the FIFO
 * allows reached the kernel), else RINGAR_SUCCESS.  Eager calls and replays
 * of captured calls record their errors in separate words, so neither can
 * hide the other's; one call returns one error (call it again for the next).
 * After an eager call's error the FIFO state stays valid for later calls.
 * After a replay's error this call also clears the counters and line flags
 * the captured form expects to find at zero (the replay that gave up left
 * some behind), so the graph may be replayed again; call it once the replay
 * has completed (synchronise the stream it was replayed on first).
 * RINGAR_ERR_DEVICE if a HIP call fails. */
ringar_result_t ringar_get_async_error(ringar_stream_t stream);

/* Resource cleanup, the analogue of ncclCommDestroy ([BOOK] §1.4: free the
 * local resources once nothing uses them any more).  Synchronises every
 * device the library has used and frees every FIFO, counter and error word
 * it allocated (they are re-created on the next call).  Graphs captured
 * before this call hold freed addresses: do not replay them.  Returns
 * RINGAR_ERR_DEVICE if a HIP call fails. */
ringar_result_t ringar_release(void);

/* Static text naming a result code (the error classes of [BOOK] Japanese
 * edition ch. 5-6: invalid argument, invalid usage, internal error); never
 * NULL, "unknown result" for codes outside the enum. */
const char* ringar_result_string(ringar_result_t r);

/* Text of the last HIP error or refusal reason seen by this thread ("" if
 * none); valid until this thread's next call into the library. */
const char* ringar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGAR_H */
