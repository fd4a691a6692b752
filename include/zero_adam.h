/*
 * zero_adam.h: C ABI of the fused ZeRO-sharded Adam step for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the one defined by "ZeRO-Sharded Adam Step"
 * (scratchllm.com/problems/zero-sharded-optimizer), sections "The step", "The
 * shards" and "What to implement": N workers hold full-length local gradients;
 * the parameter indices are split into N shards by np.array_split; (1) a
 * reduce-scatter gives worker r the average, over the workers, of the gradient
 * entries in its own shard, (2) worker r runs Adam on its shard with its own m and v,
 * (3) an all-gather leaves the full updated parameter vector on every worker.
 * Per "Requirements" the outcome matches ordinary Adam over the whole vector
 * driven by the averaged gradient. Stages and memory follow "Data parallelism and ZeRO
 * stages 1 to 3" (openlearn L11.3), sections "2. Principles" and "4. The
 * interface".
 *
 * On one GPU every logical worker lives in the same HBM, so the reduce-scatter
 * is a local sum over N gradient buffers (in rank order, left to right) and the
 * all-gather is the store into the one gathered parameter buffer. The whole
 * step is one kernel launch that streams each byte through HBM once (a call
 * longer than 2^32 elements is enqueued as consecutive launches of at most
 * 2^32 elements each, on offset views of the same buffers).
 *
 * Per element, in the state type S (double in fp64 mode, float otherwise),
 * each operation one IEEE round-to-nearest-even operation, never fused:
 *     gb  = (g_0 + g_1 + ... + g_{N-1}) / N
 *     m   = b1*m + (1-b1)*gb
 *     v   = b2*v + (1-b2)*(gb*gb)
 *     mh  = m / (1-b1^t);   vh = v / (1-b2^t)
 *     den = sqrt(vh) + eps
 *     w   = w * (1 - lr*wd)                  where decay applies
 *     w   = w - lr*(mh/den)
 * 1-b1, 1-b2, 1-b1^t, 1-b2^t and 1-lr*wd are formed in double on the host and
 * rounded once to S. In mixed mode the gathered parameter is the bf16 (or
 * fp16) round-to-nearest-even of w (NaN stored as 0x7FC0, or 0x7E00).
 *
 * Conventions shared by every function:
 *   - All device buffers are owned by the caller; the library never allocates,
 *     frees or keeps device memory, and keeps no pointer after a call returns.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and runs asynchronously; synchronisation is the caller's job.
 *     Calls that overlap in time on buffers they both write race.
 *   - Every argument is validated on the host before any HIP call; a rejected
 *     call enqueues nothing. No exception crosses the ABI.
 *   - A non-OK status leaves a message for zero_last_error() in the calling
 *     thread.
 */
#ifndef ZERO_ADAM_H
#define ZERO_ADAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZERO_OK = 0,
  ZERO_EINVAL = -1,       /* a bad argument; nothing was enqueued */
  ZERO_EUNSUPPORTED = -2, /* valid, but outside what this library implements */
  ZERO_EHIP = -3          /* the HIP runtime reported an error at launch; in a
                             call of several launches (buckets, pieces of 2^32
                             elements, the clipped step) the ones before it
                             may already be enqueued */
} zero_status;

typedef enum {
  /* fp64 parameters, gradients, m and v; the parameter is its own master. */
  ZERO_MODE_F64 = 0,
  /* fp32 parameters, gradients, m and v (K = 8 optimizer bytes per parameter,
   * "ZeRO One: Sharding the Optimizer", section "Training Memory
   * Requirements"); the parameter is its own master. */
  ZERO_MODE_F32 = 1,
  /* bf16 parameters and gradients, fp32 master, m and v (K = 12, same section;
   * "Data Parallelism & ZeRO", section "ZeRO, stage by stage"). */
  ZERO_MODE_MIXED_BF16 = 2,
  /* IEEE fp16 parameters and gradients, fp32 master, m and v (K = 12; "Data
   * parallelism and ZeRO optimization", section "Memory Consumption
   * Analysis"). The gathered parameter is the fp16 round-to-nearest-even of w,
   * with gradual underflow and overflow to infinity (NaN stored as 0x7E00). */
  ZERO_MODE_MIXED_F16 = 3
} zero_mode;

typedef enum {
  /* Bias-corrected Adam with decoupled (AdamW) weight decay, as above. */
  ZERO_OPT_ADAM = 0,
  /* Momentum SGD, the other optimizer "Data parallelism and ZeRO stages 1 to
   * 3" wraps (M10.2 SGD, run with momentum in its DDP tests); no formula is
   * printed, so it follows torch.optim.SGD, per element in S, never fused:
   *     d = gb;  where decay applies: d = d + wd*w        (coupled L2 decay)
   *     if momentum != 0:
   *       buf = (t == 1) ? d : momentum*buf + (1-dampening)*d
   *       d   = nesterov ? d + momentum*buf : buf
   *     w = w - lr*d
   * The momentum buffer is states.m; states.v is not used (may be NULL);
   * beta1, beta2 and eps are ignored. 1-dampening is formed in double and
   * rounded once to S. */
  ZERO_OPT_SGD = 1
} zero_optimizer;

/* Largest number of workers one zero_step call accepts (the gradient pointers
 * travel in the kernel's argument block). zero_shard_bounds and
 * zero_memory_bytes accept any N >= 1. */
#define ZERO_MAX_WORKERS 256

/* Hyperparameters and the shape of one call. There are no hidden defaults:
 * every field is used as given ("Data parallelism and ZeRO stages 1 to 3",
 * section "5. Pitfalls", dropped hyperparameters). */
typedef struct {
  int64_t n;         /* parameters in the gathered vector; 1 <= n <= 2^56 */
  int32_t n_workers; /* N, 1 <= N <= ZERO_MAX_WORKERS for zero_step; N > n is
                        allowed and gives trailing empty shards */
  int32_t rank;      /* -1: every worker's share in this call (full mode);
                        0..N-1: only worker `rank`'s share (rank mode) */
  int32_t mode;      /* a zero_mode */
  int32_t optimizer; /* a zero_optimizer */
  double lr;         /* finite */
  double beta1;      /* Adam: in [0, 1) */
  double beta2;      /* Adam: in [0, 1) */
  double eps;        /* Adam: finite, > 0 */
  double weight_decay; /* finite, >= 0; 0 disables decay (decoupled for Adam,
                          coupled L2 for SGD) */
  /* Optional device bitmask over the global index space [0, n): element i
   * decays iff bit (i % 32) of word i / 32 is set. It must hold at least
   * (n + 31) / 32 readable words and be 4-byte aligned. NULL: every element
   * decays when weight_decay > 0. Ignored when weight_decay == 0. */
  const uint32_t* wd_mask;
  double momentum;   /* SGD: finite, >= 0; 0 keeps no buffer */
  double dampening;  /* SGD: in [0, 1] */
  int32_t nesterov;  /* SGD: 0 or 1; 1 needs momentum > 0 and dampening == 0 */
  int32_t reserved;  /* must be 0 */
} zero_hparams;

/* Optimizer state, caller-owned device buffers, each 16-byte aligned.
 *   (SGD: m is the momentum buffer and v is unused and may be NULL.)
 *   Full mode (rank == -1): m and v hold n elements of S; worker r's shard is
 *     the view [a_r, b_r) of each (the N per-worker (m_shard, v_shard) pairs of
 *     "What to implement", laid back to back). master holds n fp32 values in
 *     the mixed modes and must be NULL in fp64/fp32 mode, where the parameter is
 *     updated in place and is its own master.
 *   Rank mode (rank == r): m, v and master each hold c_r = b_r - a_r elements
 *     of S: only worker r's shard. master is required in every mode (the rank's
 *     master copy of its chunk, "Data parallelism and ZeRO stages 1 to 3",
 *     section "2. Principles", stage 1). */
typedef struct {
  void* master;
  void* m;
  void* v;
} zero_states;

/* init_states ("What to implement"): zero m and v, and set the master copy
 * from the parameters (exact bf16/fp16 -> fp32 widening in the mixed modes, a copy in
 * rank mode's fp64/fp32 master). `param` is the gathered parameter vector of n
 * elements (bf16/fp16 in the mixed modes, else S), read-only; in rank mode only
 * [a_r, b_r) of it is read. Enqueued on `stream`. An empty rank shard
 * enqueues nothing and touches no buffer (they may be NULL). Errors as for
 * zero_step, without the step scalars and t. */
zero_status zero_init_states(const zero_hparams* hp, const void* param,
                             const zero_states* states, void* stream);

/* zero_step ("What to implement"; "The step" items 1-3): one fused step.
 *   param: the gathered parameter vector, n elements (bf16/fp16 in the mixed modes,
 *     else S), updated in place. Full mode: every element is rewritten; it
 *     must be 16-byte aligned. Rank mode: only [a_r, b_r) is written; it must
 *     be aligned to its element size.
 *   grads: host array of N device pointers, in rank order, read-only, each
 *     16-byte aligned (elements of G = bf16/fp16 in the mixed modes, else S). Full mode:
 *     worker k's full local gradient, n elements. Rank mode: the chunk
 *     g_k[a_r:b_r) that worker k contributes to shard r, c_r elements.
 *     Gradient buffers may alias one another but not any buffer the step
 *     writes.
 *   states: as described at zero_states; updated in place.
 *   t: the 1-based step number ("What to implement"); t < 1 is rejected.
 * Rank mode with an empty shard (c_r == 0) is valid and enqueues nothing; then
 * no buffer is touched and param, grads and states may be NULL (the scalar
 * arguments and t are still checked).
 * Errors: ZERO_EINVAL for a null or misaligned pointer, overlapping written
 * ranges, n outside [1, 2^56], N outside [1, ZERO_MAX_WORKERS], rank outside [-1, N), t < 1,
 * a non-finite scalar, a beta outside [0, 1), eps <= 0, weight_decay < 0, an
 * unknown optimizer, SGD momentum < 0, dampening outside [0, 1], nesterov
 * without momentum or with dampening, a mode/master mismatch, or
 * reserved != 0; ZERO_EHIP if the launch fails. */
zero_status zero_step(const zero_hparams* hp, void* param, const void* const* grads,
                      const zero_states* states, int64_t t, void* stream);

/* The step on the sub-range [begin, end) of the call's index space (full mode:
 * [0, n); rank mode: [0, c_r) of worker `rank`'s shard), with the same
 * full-length buffers and arguments as zero_step. The step is elementwise
 * ("Data parallelism and ZeRO stages 1 to 3", section "2. Principles"), so
 * stepping disjoint ranges that cover the index space, in any order and on any
 * streams, gives bit for bit the result of one zero_step. This is the
 * bucketed step: gradients reduced bucket by bucket during backward
 * ("Data Parallelism & ZeRO", section "Data parallelism, and why the obvious
 * implementation is bad": ~25 MB buckets) can be stepped as each bucket lands.
 * begin must be a multiple of 8 (keeps every stream's groups aligned); end may
 * be anything up to the range's length. Errors as zero_step, plus ZERO_EINVAL
 * for a bad range; an empty range enqueues nothing. */
zero_status zero_step_range(const zero_hparams* hp, void* param, const void* const* grads,
                            const zero_states* states, int64_t t, int64_t begin, int64_t end,
                            void* stream);

/* The bucketed step in one call: for i = 0 .. nbuckets-1 in that order, bucket
 * i covers [edges[2i], edges[2i+1]) of the call's index space (the begin a
 * multiple of 8, as for zero_step_range) and, when ready_events is non-NULL and
 * ready_events[i] (a hipEvent_t) is non-NULL, is launched on `stream` only after
 * that event completes. This is the overlap of the step with backward ("Data
 * Parallelism & ZeRO", section "Data parallelism, and why the obvious
 * implementation is bad": gradients reduced in ~25 MB buckets while backward
 * runs): the producer records one event per bucket as its gradients land, and
 * the step of each bucket starts as soon as they have, with no host round trip
 * per bucket. The buckets must be disjoint (they need not cover the range); each
 * element of a bucket then ends bit for bit as after zero_step. Every argument
 * and every bucket is validated before anything is enqueued; an invalid bucket
 * enqueues nothing. Errors as zero_step_range, plus ZERO_EINVAL for
 * nbuckets < 0, NULL edges or overlapping buckets; ZERO_EHIP if a wait or
 * launch fails (buckets before it stay enqueued). */
zero_status zero_step_buckets(const zero_hparams* hp, void* param, const void* const* grads,
                              const zero_states* states, int64_t t, const int64_t* edges,
                              int32_t nbuckets, void* const* ready_events, void* stream);

/* ---- Step scalars in device memory, for captured launches -----------------
 * zero_step and zero_step_range bake the step-dependent scalars (1 - b1^t,
 * 1 - b2^t, and for SGD whether t == 1) into the launch. A launch captured
 * into a HIP graph would then replay step t forever. zero_step_range_dev
 * takes them from a small device buffer instead, so one captured launch (or
 * a captured sequence of buckets) serves every step: before each replay the
 * caller writes the next step's scalars into that buffer. */

/* The step-dependent scalars of step t; 24 bytes, 8-byte aligned. */
typedef struct {
  double bias1; /* 1 - beta1^t, formed in double */
  double bias2; /* 1 - beta2^t, formed in double */
  int64_t t;    /* the 1-based step number */
} zero_step_scalars;

/* Host-only; touches no device. Fills *out for step t exactly as zero_step
 * forms these values. Errors as zero_step for the hyperparameters and t. */
zero_status zero_step_scalars_fill(const zero_hparams* hp, int64_t t, zero_step_scalars* out);

/* zero_step_range with the step's scalars read by the kernel from
 * dev_scalars: a device pointer (8-byte aligned, not overlapping any buffer
 * the step writes) holding the zero_step_scalars that zero_step_scalars_fill
 * produced for the step being run. The host validates everything else as for
 * zero_step_range (with t = 1); the device values are used as given, so the
 * buffer must hold a filled value whenever the launch runs. The result is bit
 * for bit that of zero_step_range with the same t. For graph capture
 * (hipStreamBeginCapture, or torch.cuda.graph): the call enqueues one kernel
 * (one per 2^32 elements) and makes no allocation, copy, set or
 * synchronisation. */
zero_status zero_step_range_dev(const zero_hparams* hp, void* param, const void* const* grads,
                                const zero_states* states, const zero_step_scalars* dev_scalars,
                                int64_t begin, int64_t end, void* stream);

/* ---- The materialised reduce-scatter mean and global-norm clipping ----------
 * "Data parallelism and ZeRO stages 1 to 3", section "2. Principles": stage 1
 * keeps the averaged gradient in .grad ("Your emulation's bookkeeping"), and
 * the reduce-scatter of stage 2 leaves each rank its chunk of it; section
 * "Going further": sharded global-norm clipping sums the chunks'
 * squared norms across ranks ahead of the update. The clipping factor is
 * min(1, max_norm / (sqrt(sumsq) + 1e-6)) in double (the definition torch's
 * clip_grad_norm_ uses), rounded once to S and multiplied into the mean
 * gradient before the moments. The squared norm is summed in double in a fixed
 * order that depends only on n and the mode (block sums, then the blocks in
 * order), so it is the same on every run; it may differ from another summation
 * order in the last bits. */

/* zero_step that also stores the averaged gradient ("Data parallelism and ZeRO
 * stages 1 to 3", section "2. Principles": in stage 1 each rank keeps the full
 * averaged gradient in .grad, "Your emulation's bookkeeping"). In the same pass
 * over the gradients, mean_out[j] receives gb = (g_0 + ... + g_{N-1}) / N of
 * each element j of the call (full mode: n elements; rank mode: the c_r
 * elements of worker `rank`'s shard), in S, bit for bit the value the update
 * uses and the one zero_mean_grad computes. It costs sizeof(S) more bytes per
 * parameter than zero_step, against N*sizeof(G) + sizeof(S) for a separate
 * zero_mean_grad pass. Every other output is bit-identical to zero_step's.
 * mean_out: device, 16-byte aligned, must not overlap any buffer the step reads
 * or writes. Errors as zero_step, plus ZERO_EINVAL for a NULL, misaligned or
 * overlapping mean_out (unless the rank's shard is empty: then nothing is
 * touched). */
zero_status zero_step_with_mean(const zero_hparams* hp, void* param, const void* const* grads,
                                const zero_states* states, int64_t t, void* mean_out,
                                void* stream);

/* Device workspace bytes zero_mean_grad needs when sumsq_out is non-NULL. */
zero_status zero_mean_grad_workspace_bytes(const zero_hparams* hp, size_t* bytes);

/* The reduce-scatter mean of the call's range, materialised: mean_out[j] for
 * the call's elements (full mode: n; rank mode: c_r of worker `rank`, from its
 * N chunk gradients), in S, computed exactly as zero_step computes it (rank-order
 * left fold, one division by N). If sumsq_out is non-NULL (a device double),
 * also writes the range's squared norm sum(mean^2) there, using `workspace`
 * (16-byte aligned, >= zero_mean_grad_workspace_bytes). In rank mode that is
 * this shard's squared norm: the caller sums the ranks' values (the all-reduce)
 * before zero_step_mean. mean_out is 16-byte aligned and must not overlap the
 * gradients, the workspace or sumsq_out. Only hp's shape fields are used.
 * Errors as zero_step. */
zero_status zero_mean_grad(const zero_hparams* hp, const void* const* grads, void* mean_out,
                           double* sumsq_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * zero_mean_grad with no workspace argument. The squared norm's per-block
 * partial sums go to a library-owned static device array of 16 MiB (2^21
 * doubles) that each GPU the library runs on holds until the process ends; its
 * device address is looked up on the first call on each device. The call
 * allocates nothing and calls no allocating routine. Results are bit for bit
 * those of zero_mean_grad. Every call on one GPU shares that GPU's array:
 * calls with sumsq_out non-NULL that overlap in time on one GPU (on different
 * streams, or captured into graphs replayed concurrently) race on it and must
 * be ordered by the caller. The array needs no clearing: each call writes
 * every partial it reads. Limit: the call's range may need at most 2^21
 * partial sums, which is 2^33 elements in fp32 and the mixed modes and
 * 2^30 + 1 in fp64; a larger range with sumsq_out non-NULL returns ZERO_EINVAL (use
 * zero_mean_grad with a workspace). With sumsq_out NULL the scratch is not
 * used and any size is accepted. Other errors as zero_mean_grad; ZERO_EHIP
 * also if the scratch's address cannot be looked up. */
zero_status zero_mean_grad_noalloc(const zero_hparams* hp, const void* const* grads,
                                   void* mean_out, double* sumsq_out, void* stream);

/* The step driven by a materialised mean gradient (mean_grad: the call's len
 * elements of S, 16-byte aligned, read-only), otherwise as zero_step. If
 * clip_sumsq is non-NULL it points to the global squared norm (device double,
 * 8-byte aligned, not inside any buffer the step writes) and the mean is
 * scaled by the clipping factor for max_norm (finite, > 0).
 * Unclipped, or with a factor of exactly 1, the result is bit-identical to
 * zero_step on the gradients that produced the mean. */
zero_status zero_step_mean(const zero_hparams* hp, void* param, const void* mean_grad,
                           const zero_states* states, int64_t t, const double* clip_sumsq,
                           double max_norm, void* stream);

/* Device workspace bytes zero_step_clipped needs: the mean gradient (n values
 * of S), the block partial sums and the squared norm. */
zero_status zero_step_clipped_workspace_bytes(const zero_hparams* hp, size_t* bytes);

/* One clipped step, full mode: the materialised mean, its global squared norm
 * (also written to sumsq_out if non-NULL), and the step with the clipping
 * factor for max_norm, all enqueued on `stream`. Rank mode returns
 * ZERO_EUNSUPPORTED: a rank alone does not hold the other shards' norms (use
 * zero_mean_grad, sum the ranks' squared norms, then zero_step_mean). The
 * workspace (16-byte aligned, >= zero_step_clipped_workspace_bytes) and
 * sumsq_out must not overlap any buffer the step reads or writes. */
zero_status zero_step_clipped(const zero_hparams* hp, void* param, const void* const* grads,
                              const zero_states* states, int64_t t, double max_norm,
                              double* sumsq_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Per-rank memory in bytes ("Data parallelism and ZeRO stages 1 to 3",
 * section "2. Principles", table and "Your emulation's bookkeeping"; "Data
 * Parallelism & ZeRO", section "ZeRO, stage by stage"; "Data parallelism and
 * ZeRO optimization", sections "Memory Consumption Analysis" and "ZeRO-1/2/3";
 * "ZeRO One: Sharding the Optimizer", section "Training Memory Requirements"). */
typedef struct {
  int64_t params;
  int64_t grads;
  int64_t optimizer;
  int64_t total; /* params + grads + optimizer */
} zero_mem;

/* Host-only; touches no device. Rank `rank` of N holds the chunk of
 * c = b_r - a_r elements. Widths by mode (params P, gradient G, optimizer K
 * bytes per parameter): mixed 2, 2, 12; fp32 4, 4, 8; fp64 8, 8, 16.
 *   convention 0 (the closed forms):
 *     stage 0 (plain data parallelism): P n,  G n,  K n
 *     stage 1 (optimizer state sharded): P n,  G n,  K c
 *     stage 2 (+ gradients sharded):     P n,  G c,  K c
 *     stage 3 (+ parameters sharded):    P c,  G c,  K c
 *   convention 1 (the emulation's bookkeeping of the L11.3 byte table, one
 *   value width B = P; fp64 and fp32 modes only):
 *     stage 0 (one process): B n,  B n,        2 B n
 *     stage 1: B n,  B n + B c,  3 B c   (moments + master chunk; full mean
 *              gradients kept in .grad plus the chunk's gradient)
 *     stage 2: B n,  B c,        3 B c
 *     stage 3: B c,  B c,        2 B c   (the chunk is the parameter storage)
 * Errors: ZERO_EINVAL for n < 1 or n > 2^56, N < 1, rank outside [0, N), stage outside
 * [0, 3], an unknown mode or convention, or a NULL out; ZERO_EUNSUPPORTED for
 * convention 1 in the mixed modes. */
zero_status zero_memory_bytes(int64_t n, int32_t n_workers, int32_t rank, int32_t stage,
                              int32_t mode, int32_t convention, zero_mem* out);

/* The smallest ZeRO stage that fits ("Data parallelism and ZeRO optimization",
 * section "When to Use Each ZeRO Stage": the minimum stage whose memory need is
 * below the memory available). For stage s in 0, 1, 2, 3 the need is
 * zero_memory_bytes(n, N, 0, s, mode, 0).total (rank 0 holds the largest shard)
 * plus activation_bytes; *stage is the first s whose need is < available_bytes,
 * or -1 when none is. Host-only. Errors: ZERO_EINVAL for n outside [1, 2^56], N < 1, an
 * unknown mode, a negative byte count or a NULL stage. */
zero_status zero_min_stage(int64_t n, int32_t n_workers, int32_t mode, int64_t activation_bytes,
                           int64_t available_bytes, int32_t* stage);

/* Shard r of np.array_split(np.arange(n), N) as the half-open range
 * [*begin, *end) ("ZeRO-Sharded Adam Step", section "The shards"): the first
 * n mod N shards hold floor(n/N) + 1 indices, the rest floor(n/N). Host-only.
 * n >= 0 (n == 0 gives empty shards), N >= 1, 0 <= r < N; else ZERO_EINVAL. */
zero_status zero_shard_bounds(int64_t n, int32_t n_workers, int32_t r, int64_t* begin,
                              int64_t* end);

/* The calling thread's message for its last non-OK status ("" if none). The
 * pointer stays valid until the thread's next call into the library. */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_ADAM_H */
