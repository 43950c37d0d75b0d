/*
 * ra.h — C-ABI of libra: one device's share of Ring Attention on an AMD Instinct MI355X
 * (gfx950), in hand-written HIP.
 *
 * The method (Ring Attention with Blockwise Transformers):
 *   Device i of an N-device ring keeps its query shard Q_i (L = S/N tokens) resident while
 *   the N key/value shards pass by in ring order; at ring step k it holds the KV shard of
 *   device (i - k) mod N (page 4, "The Ring Communication Protocol").  It attends Q_i to
 *   each shard as it arrives, carrying the online-softmax state across steps (page 1,
 *   "Blockwise Attention and Online Softmax Formulations"), and the result equals plain
 *   softmax attention over the whole sequence.  Causal masking is by global token
 *   position, under one of three sequence layouts (page 1, "Causal Masking Dynamics:
 *   Striped Attention and Zig-Zag Topologies").  Grouped-query attention shares each KV
 *   head between h / n_kv consecutive query heads (page 3, section 2).
 *
 * Conventions for every entry point:
 *   - Pointers named q, k, v, o, lse, ws, ... are DEVICE pointers owned by the caller,
 *     16-byte aligned.  The library never allocates or frees device memory (the one fixed
 *     array of ra_ring_fwd_noalloc is part of the loaded library, not an allocation).
 *   - Streams are hipStream_t values passed as ra_stream (NULL = the null stream).  Calls
 *     only enqueue work and return; they never synchronise (except ra_ring_fwd_timed).
 *   - Every argument is validated before anything is enqueued; on any error nothing is
 *     written and a negative ra_status is returned, with detail in ra_last_error().
 *   - Tensor layouts (row-major, innermost last), matching the pages' (batch, seq_block,
 *     heads, head_dim) layout (page 1, "Practical Implementation Patterns"):
 *         q, o, dout           [b][L][h][d]
 *         k, v (one shard)     [b][L][n_kv][d]
 *         k_all, v_all         [N][b][L][n_kv][d]   shard j in its own local order
 *         lse, delta           [b][h][L]            fp32
 *   - LSE is the natural-log softmax denominator of each query row, in units of the scaled
 *     logit: LSE = m + ln(sum_j exp(s_j - m)), s_j = scale * q.k_j.  A row with no
 *     allowed key has LSE = -inf and O = 0.
 *   - Thread safety: calls are reentrant; the only global state is the per-device scratch
 *     array and events of ra_ring_fwd_noalloc, set up once under a lock (see there).
 *   - Debugging aid: with RA_POISON_STAGING=1 in the environment, the ring passes
 *     (ra_ring_fwd[_timed], ra_ring_bwd[_timed], ra_ring_bwd_kv_stationary) fill each staging
 *     buffer with NaN on the copy stream as soon as the step that read it has finished, so a
 *     step reading a buffer outside the window between its copy and its consumption yields
 *     NaN.  Off by default; it adds one fill per staged step.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ra_status;
#define RA_OK 0
#define RA_ERR_INVALID_ARG (-1) /* bad shape, index, enum, null or misaligned pointer   */
#define RA_ERR_UNSUPPORTED (-2) /* valid problem with no kernel (e.g. bf16 with d != 128, or a
                                 bf16 K/V slice L*n_kv*d*2 of 2 GiB or more)               */
#define RA_ERR_WORKSPACE (-3)   /* workspace smaller than ra_ring_{fwd,bwd}_workspace()  */
#define RA_ERR_HIP (-4)         /* a HIP call or launch failed                            */

/* Sequence layouts (page 1, "Causal Masking Dynamics"; page 3, section 6). */
#define RA_LAYOUT_CONTIGUOUS 0 /* shard p holds tokens [pL, pL+L)                             */
#define RA_LAYOUT_STRIPED 1    /* token t lives on shard t mod N (local index t div N)          */
#define RA_LAYOUT_ZIGZAG 2     /* 2N chunks of L/2; shard p holds chunk p then chunk 2N-1-p     */

/* Element types of q, k, v, o (and dout). */
#define RA_F32 0
#define RA_BF16 1

/* The problem, after the pages' problem statement: Q/K/V shapes, ring size N, causal
 * flag and sharding layout.  All sizes are per shard; the sequence length is S = N * L. */
typedef struct ra_problem {
  int32_t b;      /* batch                                                        */
  int32_t L;      /* tokens per shard (>= 1; even for zigzag)                      */
  int32_t h;      /* query heads                                                   */
  int32_t n_kv;   /* key/value heads; h % n_kv == 0; query head hq reads hq/(h/n_kv) */
  int32_t d;      /* head dimension: bf16 supports 128; fp32 supports 64 and 128    */
  int32_t N;      /* ring size = number of shards (>= 1)                           */
  int32_t causal; /* 0 or 1                                                        */
  int32_t layout; /* RA_LAYOUT_*; only matters when causal = 1                      */
  int32_t dtype;  /* RA_F32 or RA_BF16                                             */
  float scale;    /* softmax scale on q.k; <= 0 selects 1/sqrt(d)                   */
  /* Packed documents (page 3, section 5: documents packed end to end into one window, a
   * block-diagonal mask stopping attention across them).  Both NULL: one sequence.
   * Otherwise DEVICE arrays [b][L] of int32 giving, for every query row of the shard the
   * call computes, the global position of its document's first token (doc_begin) and one
   * past its last (doc_end); the row attends only to keys at positions in
   * [doc_begin, doc_end), and only to those at or before its own position when causal.
   * Both must be nondecreasing along the shard's rows, as they are for packed documents
   * (ra_document_ranges builds them).  They are read on the device and not validated: bad
   * values give wrong masks, never out-of-bounds accesses.  Both or neither. */
  const int32_t* doc_begin;
  const int32_t* doc_end;
  /* Ring steps per kernel launch of a bf16 forward pass (ra_ring_fwd, ra_ring_fwd_timed,
   * ra_ring_fwd_noalloc; other entry points ignore it).  Page 1 ("Blockwise Attention and
   * Online Softmax Formulations") carries the online-softmax state (m, l, O) from one KV
   * block to the next; page 2 ("FlashAttention Integration") merges per-step partials by
   * their LSE instead.  Both give the same result; this chooses where the state lives.
   *   1: one launch per ring step, merged into (O, LSE) in HBM after each; the KV shard of
   *      the next step is staged into the idle half of a double buffer while a step runs.
   *   m >= 2: step 0 (the local shard) alone, then the other steps m at a time, each launch
   *      walking its KV shards in ring order with the state on chip and merging once; every
   *      remote shard is staged into a slot of its own (ra_ring_fwd_workspace grows to
   *      2 (N - 1) K/V slots), each launch waiting only for the copies of its own shards.
   *   0: the library's choice for N >= 3 when the workspace holds the slots: all N - 1
   *      remote steps in one launch when b h L^2 <= 2^33 (short steps) or with packed
   *      documents, else up to 4 steps per launch; 1 when the slots do not fit.
   * On a real ring a device forwards each shard as it arrives, so a launch of m steps after
   * step 0 finds its shards staged when m transfers take no longer than step 0's compute. */
  int32_t steps_per_launch;
} ra_problem;

typedef void* ra_stream; /* a hipStream_t */

/* ---------------------------------------------------------------------------------------
 * ra_step_fwd — one ring step.
 * Attends shard q_shard's queries to the single KV shard kv_shard (the block a device
 * holds at one step of the ring; page 1, "The Ring Attention Protocol"), masked by global
 * positions when causal.  Writes the step's normalised partial: o_part [b][L][h][d] fp32
 * and lse_part [b][h][L] fp32; rows with no allowed key in this shard get (0, -inf).
 * q is [b][L][h][d] and k, v are [b][L][n_kv][d] in p->dtype.
 * ------------------------------------------------------------------------------------- */
ra_status ra_step_fwd(const ra_problem* p, int32_t q_shard, int32_t kv_shard, const void* q,
                      const void* k, const void* v, float* o_part, float* lse_part,
                      ra_stream stream);

/* ---------------------------------------------------------------------------------------
 * ra_merge_lse — combine a step's partial into the running result, in place.
 * Page 2, "FlashAttention Integration": partial outputs are rescaled to the new maximum
 * and summed; page 3, section 3: the whole state must be carried, not O alone.  In
 * (O, LSE) form:  lse = ln(exp(lse_acc) + exp(lse_part)) (computed around the maximum),
 * o_acc = exp(lse_acc - lse) o_acc + exp(lse_part - lse) o_part.  (0, -inf) is the
 * identity: start the accumulator at o_acc = 0, lse_acc = -inf.  All fp32;
 * o_acc, o_part [b][L][h][d]; lse_acc, lse_part [b][h][L].  p->dtype is ignored.
 * ------------------------------------------------------------------------------------- */
ra_status ra_merge_lse(const ra_problem* p, float* o_acc, float* lse_acc, const float* o_part,
                       const float* lse_part, ra_stream stream);

/* ---------------------------------------------------------------------------------------
 * ra_finalize — write the merged fp32 output o_acc [b][L][h][d] in p->dtype (bf16 round to
 * nearest even, or an fp32 copy) to o (page 1: the final output after the last step).
 * ------------------------------------------------------------------------------------- */
ra_status ra_finalize(const ra_problem* p, const float* o_acc, void* o, ra_stream stream);

/* Bytes of device workspace for ra_ring_fwd (each part 256-byte aligned).  With ring steps
 * batched into launches (p->steps_per_launch >= 2, or 0 for a bf16 ring of N >= 3): a K/V
 * slot for each of the N - 1 remote shards and the fp32 output accumulator [b][L][h][d].
 * With one launch per step: two KV staging buffers (the double buffer of page 1, "Practical
 * Implementation Patterns") and, unless dtype is fp32, the fp32 output accumulator.  Either
 * way, for bf16 without packed documents and L <= 4096, then a second fp32 accumulator
 * [b][L][h][d] with its LSE [b][h][L].  Given less than the batched size (without the
 * second accumulator), the library's choice (0) runs one launch per step.  With the second
 * accumulator the launches of short shards may run the key range of a heavy query block as
 * two workgroups (in a batched launch, each of its KV shards' ranges in two halves), one
 * merging into each accumulator, and the pass folds the two together at the end (page 2,
 * "FlashAttention Integration": partials over disjoint key sets merge by their LSE); this
 * evens out the causal imbalance between query blocks and fills the chip when a launch has
 * few blocks.  A workspace without the second accumulator is accepted too: the pass then
 * runs every block whole (the same result up to the order of the fp32 sums).  Returns 0 if
 * p is invalid. */
size_t ra_ring_fwd_workspace(const ra_problem* p);

/* ra_fwd_step_plan — how one bf16 forward step of a pass with the second accumulator
 * distributes its query blocks over workgroups (inspection and tests; no GPU call).  Query
 * block i holds rows [i R, (i+1) R) (R = *block_rows) of the query heads of one KV head that
 * one workgroup runs; work item j (launch order; each item runs once per KV head and batch
 * row) is block[j] whole (part[j] = -1) or the first (0) or second (1) half of its key tiles.
 * Items are ordered by decreasing work.  n_cu: compute units to plan for.  Writes up to
 * max_items entries of block and part and the item count to *n_items.  RA_ERR_UNSUPPORTED
 * unless dtype is bf16. */
ra_status ra_fwd_step_plan(const ra_problem* p, int32_t q_shard, int32_t kv_shard, int32_t n_cu, int32_t* block,
                           int32_t* part, int32_t max_items, int32_t* n_items, int32_t* block_rows);

/* ---------------------------------------------------------------------------------------
 * ra_ring_fwd — the whole forward ring pass of device q_shard.
 * Step k = 0..N-1 attends q to KV shard (q_shard - k) mod N and merges the partial into the
 * running (O, LSE); the final o [b][L][h][d] (p->dtype) and lse [b][h][L] (fp32) equal
 * plain softmax attention of q over the whole sequence.  The KV shards of the remote steps
 * are copied on the `copy` stream while earlier steps compute on `compute` (the ring's
 * receive from the previous device, emulated on one GPU; page 1, "The Ring Attention
 * Protocol and Overlapped Communication"): into the idle half of a double buffer, one step
 * ahead, with one launch per step, or each into a slot of its own when steps are batched
 * into launches (ra_problem.steps_per_launch).  Step 0 reads the local shard in place.
 * Steps whose KV shard is entirely in the causal future are skipped (their copy still
 * runs).  With bf16 the last live step writes o itself, rounded to
 * nearest even (no separate finalize pass).  `copy` may be NULL or equal to `compute`
 * (copies then run in order on `compute`).  All work has finished when work queued on `compute` after this
 * call runs.  ws must hold ra_ring_fwd_workspace(p) bytes, or those less the second
 * accumulator (see there).
 * ------------------------------------------------------------------------------------- */
ra_status ra_ring_fwd(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                      const void* v_all, void* o, float* lse, void* ws, size_t ws_bytes,
                      ra_stream compute, ra_stream copy);

/* Per-step timings reported by ra_ring_fwd_timed (and ra_ring_bwd), in milliseconds from an
 * event recorded on `compute` at entry.  A launch that runs ring steps k .. k + n - 1 is
 * timed at step k (step_begin_ms, step_end_ms) with launch_steps[k] = n; the other steps'
 * entries are -1 and 0, as are those of skipped steps; copy times are -1 where no copy ran. */
#define RA_MAX_TIMED_STEPS 64
typedef struct ra_ring_timing {
  int32_t n_steps;
  float step_begin_ms[RA_MAX_TIMED_STEPS];
  float step_end_ms[RA_MAX_TIMED_STEPS];
  float copy_begin_ms[RA_MAX_TIMED_STEPS]; /* copy that stages the KV of step k */
  float copy_end_ms[RA_MAX_TIMED_STEPS];
  float total_ms;
  int32_t launch_steps[RA_MAX_TIMED_STEPS];
} ra_ring_timing;

/* ra_ring_fwd_timed — ra_ring_fwd with timing events around every step kernel (on
 * `compute`) and every staging copy (on `copy`).  Same results as ra_ring_fwd; unlike every
 * other entry point it synchronises `compute` before returning.  Requires N <= 64.  For
 * measurement (per-step compute time, copy/compute overlap); t is a host pointer. */
ra_status ra_ring_fwd_timed(const ra_problem* p, int32_t q_shard, const void* q,
                            const void* k_all, const void* v_all, void* o, float* lse, void* ws,
                            size_t ws_bytes, ra_stream compute, ra_stream copy,
                            ra_ring_timing* t);

/* ---------------------------------------------------------------------------------------
 * ra_ring_fwd_noalloc — ra_ring_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * pass, kernels and results as ra_ring_fwd, with its workspace (the KV staging buffers or
 * slots and the fp32 output accumulator) held in a fixed device array of RA_NOALLOC_SCRATCH_BYTES
 * inside the library instead of a caller buffer; the caller passes inputs and outputs only.
 * Runs on the calling thread's current device.  Each device holds its own array from the
 * library's load until the process ends; the first call on a device looks up the array's
 * address and creates the pass's events (no device memory is allocated then or later).
 * Errors: as ra_ring_fwd, and RA_ERR_WORKSPACE (nothing enqueued) when the workspace of one
 * launch per step without its second accumulator exceeds RA_NOALLOC_SCRATCH_BYTES (for bf16
 * that is 4 b L n_kv d 2 + 4 b L h d bytes plus alignment: L = 2048 with h = 32, n_kv = 8,
 * d = 128 fits), or when steps_per_launch >= 2 asks for slots that do not fit.  Under the
 * library's choice the batched steps run when their slots fit (L = 2048 with h = 32,
 * n_kv = 8, N = 4; L = 1024 with N = 8), with the second accumulator behind them when that
 * fits too (L = 1024 with h = 32, n_kv = 8, N = 8), else with one launch per step the second
 * accumulator when it fits (L = 2048 with h = 16, n_kv = 8); the results equal ra_ring_fwd's
 * with a workspace of RA_NOALLOC_SCRATCH_BYTES.  Every call on one device shares that device's array and events, and the array
 * keeps the last call's contents (each pass overwrites everything it reads, so nothing
 * needs clearing): calls whose work overlaps on one device (different streams, or threads
 * not ordered by the caller) race and give wrong results, so order them, e.g. on one stream.
 * ------------------------------------------------------------------------------------- */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ra_status ra_ring_fwd_noalloc(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                              const void* v_all, void* o, float* lse, ra_stream compute, ra_stream copy);

/* ---------------------------------------------------------------------------------------
 * Backward (page 1, "The Backward Pass and Gradient Exchange"; page 4, "The Backward Pass:
 * Symmetric Ring Operation": P is recomputed from the saved statistics, dQ accumulates on
 * the query's device, dK and dV accumulate per KV block).  The gradients are the textbook
 * ones of softmax attention; with P = exp(s - LSE) (0 where masked), D = rowsum(dO * O):
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
 * dK and dV summed over the query heads of each KV group.  bf16 with d = 128 only
 * (RA_ERR_UNSUPPORTED otherwise).  Gradients are fp32.
 * ------------------------------------------------------------------------------------- */

/* ra_bwd_preprocess — delta [b][h][L] fp32 = rowsum(dout * o); o, dout [b][L][h][d]. */
ra_status ra_bwd_preprocess(const ra_problem* p, const void* o, const void* dout, float* delta,
                            ra_stream stream);

/* ra_step_bwd — one ring step of the backward: adds the contributions of shard q_shard's
 * queries against KV shard kv_shard to dq_acc [b][L][h][d] (this device's queries) and to
 * dk_acc, dv_acc [b][L][n_kv][d] (that KV shard), all fp32 and accumulated in place.  lse
 * is the forward's [b][h][L] output (natural log), delta from ra_bwd_preprocess. */
ra_status ra_step_bwd(const ra_problem* p, int32_t q_shard, int32_t kv_shard, const void* q,
                      const void* k, const void* v, const void* dout, const float* lse,
                      const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                      ra_stream stream);

/* Bytes of device workspace ra_ring_bwd asks for: two KV staging buffers and delta
 * (ra_ring_bwd_workspace_min), then, for shards of L <= 4096 without packed documents, second
 * dK and dV buffers (2 x fp32 [b][L][n_kv][d]).  With them the dK/dV kernel of a step may run
 * the query tiles of a key block as two workgroups when the key blocks leave compute units
 * idle, the second half's sums added in after the kernel; with a workspace of the minimum size
 * every key block runs whole (the same gradients up to the order of the fp32 sums).  Returns 0
 * if p is invalid. */
size_t ra_ring_bwd_workspace(const ra_problem* p);

/* Smallest workspace ra_ring_bwd accepts: two KV staging buffers plus delta (see
 * ra_ring_bwd_workspace).  Returns 0 if p is invalid. */
size_t ra_ring_bwd_workspace_min(const ra_problem* p);

/* ra_ring_bwd — the backward ring pass of device q_shard: given its q, o, dout [b][L][h][d]
 * and lse [b][h][L] from the forward, and every shard's k_all, v_all [N][b][L][n_kv][d],
 * writes dq [b][L][h][d] and dk_all, dv_all [N][b][L][n_kv][d] (fp32): this device's
 * share of the gradients, dK and dV kept per KV shard (on a real ring they travel with
 * K and V).  KV staging as in ra_ring_fwd; steps with no allowed pair are skipped. */
ra_status ra_ring_bwd(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                      const void* v_all, const void* o, const void* dout, const float* lse,
                      float* dq, float* dk_all, float* dv_all, void* ws, size_t ws_bytes,
                      ra_stream compute, ra_stream copy);

/* ra_ring_bwd plus per-step timings (as ra_ring_fwd_timed: the step of ring step k is its
 * ra_step_bwd, the copy that of its KV shard; ms from entry, -1 for skipped steps); waits
 * for the pass to finish before returning.  N <= RA_MAX_TIMED_STEPS. */
ra_status ra_ring_bwd_timed(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                            const void* v_all, const void* o, const void* dout, const float* lse,
                            float* dq, float* dk_all, float* dv_all, void* ws, size_t ws_bytes,
                            ra_stream compute, ra_stream copy, ra_ring_timing* t);

/* ra_ring_bwd_kv_stationary — the other gradient schedule (page 1, "The Backward Pass and
 * Gradient Exchange": output gradients circulate in reverse ring order while keys and
 * values stay where they are): device kv_shard keeps its k, v [b][L][n_kv][d] and, at step
 * s, holds query shard (kv_shard + s) mod N with what its gradients need, Q, dO, the
 * forward's LSE and D = rowsum(dO * O), each computed on its home device:
 *   q_all, dout_all [N][b][L][h][d] (dtype), lse_all, delta_all [N][b][h][L] (fp32).
 * Writes dk, dv [b][L][n_kv][d] (this KV shard's complete gradients) and dq_all
 * [N][b][L][h][d] (this device's contributions to every shard's dQ; on a real ring each
 * travels with its queries back home), all fp32, overwriting them.  The incoming query
 * shard is staged into the idle half of a double buffer on `copy` while the current step
 * computes, as in ra_ring_fwd; steps with no allowed pair are skipped.  Summing dq_all over
 * all N devices gives the same dQ as ra_ring_bwd.  bf16, d = 128; no packed documents
 * (RA_ERR_UNSUPPORTED: their bounds describe one query shard's rows).  Workspace:
 * ra_ring_bwd_kv_stationary_workspace(p) bytes (two staging buffers), 0 if p is invalid. */
size_t ra_ring_bwd_kv_stationary_workspace(const ra_problem* p);
ra_status ra_ring_bwd_kv_stationary(const ra_problem* p, int32_t kv_shard, const void* k, const void* v,
                                    const void* q_all, const void* dout_all, const float* lse_all,
                                    const float* delta_all, float* dq_all, float* dk, float* dv, void* ws,
                                    size_t ws_bytes, ra_stream compute, ra_stream copy);

/* ---- All-to-all sequence parallelism, one device's share (page 3, sections 4.2 and 7) ----
 * The other way of spreading attention over N devices: each device starts with one shard
 * of the sequence for every head, trades it in an all-to-all exchange for the whole
 * sequence of h/N query heads and n_kv/N KV heads, runs one attention over the whole
 * sequence, and sends each shard's rows of its heads back in a second exchange.  Needs h
 * and n_kv to be multiples of N (the pages' divisibility constraint).
 *
 * ra_ulysses_fwd computes device head_group's share on one GPU, where the N devices'
 * shards are resident: q_all [N][b][L][h][d], k_all and v_all [N][b][L][n_kv][d], shard j
 * in its own local order under p->layout (as for ra_ring_fwd).  It writes query heads
 * [head_group h/N, (head_group+1) h/N) of every shard: o_all [N][b][L][h][d] (dtype) and
 * lse_all [N][b][h][L] (fp32); other heads are left untouched, so calling it for every head
 * group fills the whole outputs, which equal ra_ring_fwd's for every shard.  The
 * exchanges are copy kernels on `stream` (gather, then attention, then scatter).
 * Workspace: ra_ulysses_fwd_workspace(p) bytes (the gathered Q, K, V of the head group, an
 * fp32 output and the LSE of the whole sequence, and the second accumulator of
 * ra_ring_fwd_workspace when the whole-sequence problem keeps one; without it the attention
 * runs unsplit), 16-byte aligned; 0 if p is invalid for this path.  RA_ERR_INVALID_ARG if h or n_kv is not a multiple of N; RA_ERR_UNSUPPORTED
 * with packed documents or where the whole-sequence problem (b, N L, h/N, n_kv/N, d) has
 * no kernel. */
size_t ra_ulysses_fwd_workspace(const ra_problem* p);
ra_status ra_ulysses_fwd(const ra_problem* p, int32_t head_group, const void* q_all, const void* k_all,
                         const void* v_all, void* o_all, float* lse_all, void* ws, size_t ws_bytes,
                         ra_stream stream);

/* ra_ulysses_fwd plus the time of its three parts (HIP events on `stream`, ms); waits for
 * the call to finish before returning. */
typedef struct ra_ulysses_timing {
  float gather_ms;  /* first exchange: Q, K, V of the head group gathered                */
  float attend_ms;  /* the attention over the whole sequence                             */
  float scatter_ms; /* second exchange: O (converted to dtype) and LSE sent back          */
  float total_ms;
} ra_ulysses_timing;
ra_status ra_ulysses_fwd_timed(const ra_problem* p, int32_t head_group, const void* q_all,
                               const void* k_all, const void* v_all, void* o_all, float* lse_all,
                               void* ws, size_t ws_bytes, ra_stream stream, ra_ulysses_timing* t);

/* ra_ulysses_bwd — the backward of device head_group's share: gathers its heads' Q, K, V,
 * O, dO (dtype) and LSE of the whole sequence from every shard (q_all, o_all, dout_all
 * [N][b][L][h][d], k_all, v_all [N][b][L][n_kv][d], lse_all [N][b][h][L], each shard in its
 * own layout order), runs the backward of the whole-sequence attention (the same step
 * kernels as ra_step_bwd, D = rowsum(dO * O) included) and sends the gradients back: writes
 * query heads [head_group h/N, ..) of dq_all [N][b][L][h][d] and KV heads
 * [head_group n_kv/N, ..) of dk_all, dv_all [N][b][L][n_kv][d], fp32, overwriting them;
 * other heads are untouched.  With GQA a device holds every query head of its KV heads, so
 * their dK, dV are complete.  bf16, d = 128.  Workspace: ra_ulysses_bwd_workspace(p)
 * bytes, 0 if p is invalid for this path. */
size_t ra_ulysses_bwd_workspace(const ra_problem* p);
ra_status ra_ulysses_bwd(const ra_problem* p, int32_t head_group, const void* q_all, const void* k_all,
                         const void* v_all, const void* o_all, const void* dout_all, const float* lse_all,
                         float* dq_all, float* dk_all, float* dv_all, void* ws, size_t ws_bytes,
                         ra_stream stream);

/* ---- Heads and sequence cut together, one device's share (page 3, sections 7 and 8) ----
 * The two-dimensional arrangement that combines both schemes: N = N_h * N_s devices
 * (N_h = n_head_groups).  The sequence is cut into N_s ring shards of N_h L tokens under
 * p->layout (as the ring cuts it into shards); ring shard r is split into N_h consecutive
 * pieces of L tokens, and device r N_h + g holds piece g for every head (its local order).
 * Device (g, r) trades pieces with the other devices of ring shard r in an all-to-all (first
 * exchange) for the whole ring shard of head group g: query heads [g h/N_h, (g+1) h/N_h) and
 * KV heads [g n_kv/N_h, (g+1) n_kv/N_h), S/N_s tokens of h/N_h heads as page 3's table puts
 * it.  It then runs the ring of ra_ring_fwd over the N_s ring shards with the devices of head
 * group g (KV staged on `copy` as there), and sends each piece's rows back (second exchange).
 * Both dimensions must divide: N_h divides N, h and n_kv (RA_ERR_INVALID_ARG otherwise).
 *
 * ra_usp_fwd computes device (head_group, ring_rank)'s share on one GPU where the N devices'
 * inputs are resident: q_all [N][b][L][h][d], k_all and v_all [N][b][L][n_kv][d] as above.  It
 * writes query heads of head_group for devices ring_rank N_h .. ring_rank N_h + N_h - 1 of
 * o_all [N][b][L][h][d] (dtype) and lse_all [N][b][h][L] (fp32), leaving everything else; one
 * call per (head group, ring rank) fills the outputs, which equal plain attention of each
 * device's queries over the whole sequence by global position.  The other ring shards' first
 * exchanges (what the other devices of head group g gather for themselves, and the ring hands
 * over) run first in the same call.  Workspace: ra_usp_fwd_workspace(p, n_head_groups)
 * bytes (the gathered Q of the ring shard, K and V of every ring shard for the head group, an
 * fp32 output, the LSE, the ring's staging buffers and the second accumulator of
 * ra_ring_fwd_workspace when the ring problem keeps one; without it the ring runs unsplit),
 * 0 if invalid for this path.  No
 * packed documents (RA_ERR_UNSUPPORTED).  ra_usp_fwd_timed also reports the parts' times
 * (HIP events on `compute`, ms) and waits for the call to finish. */
typedef struct ra_usp_timing {
  float others_gather_ms; /* the other ring shards' first exchanges (not this device's work) */
  float gather_ms;        /* this device's first exchange                                    */
  float ring_ms;          /* the ring over the N_s ring shards                               */
  float scatter_ms;       /* the second exchange                                             */
  float total_ms;         /* gather + ring + scatter                                         */
} ra_usp_timing;
size_t ra_usp_fwd_workspace(const ra_problem* p, int32_t n_head_groups);
ra_status ra_usp_fwd(const ra_problem* p, int32_t n_head_groups, int32_t head_group, int32_t ring_rank,
                     const void* q_all, const void* k_all, const void* v_all, void* o_all, float* lse_all, void* ws,
                     size_t ws_bytes, ra_stream compute, ra_stream copy);
ra_status ra_usp_fwd_timed(const ra_problem* p, int32_t n_head_groups, int32_t head_group, int32_t ring_rank,
                           const void* q_all, const void* k_all, const void* v_all, void* o_all, float* lse_all,
                           void* ws, size_t ws_bytes, ra_stream compute, ra_stream copy, ra_usp_timing* t);

/* Host-only (no GPU work): number of (query, key) pairs shard q_shard may attend to in KV
 * shard kv_shard (or the whole sequence when kv_shard = -1), summed over the batch.  Useful
 * FLOPs of the forward are 4 * d * h * pairs (page 3, section 2: two GEMMs, 2 FLOPs per
 * multiply-add).  Returns -1 on invalid arguments. */
int64_t ra_allowed_pairs(const ra_problem* p, int32_t q_shard, int32_t kv_shard);

/* Host-only: allowed pairs as ra_allowed_pairs, with the packed-document bounds given as
 * HOST arrays [b][L] (same meaning as p->doc_begin / p->doc_end, which are ignored).
 * Returns -1 on invalid arguments. */
int64_t ra_allowed_pairs_packed(const ra_problem* p, int32_t q_shard, int32_t kv_shard,
                                const int32_t* doc_begin_host, const int32_t* doc_end_host);

/* Host-only: the per-row document bounds of shard `shard` for one batch row, from the
 * documents' global start positions bounds[0..n_docs] (bounds[0] = 0, strictly
 * increasing, bounds[n_docs] = S = N * L; all host memory).  Writes begin_out[t] and
 * end_out[t] (host arrays of L int32) for every local row t of the shard under p->layout.
 * RA_ERR_INVALID_ARG if the bounds are not of that form. */
ra_status ra_document_ranges(const ra_problem* p, int32_t shard, const int32_t* bounds,
                             int32_t n_docs, int32_t* begin_out, int32_t* end_out);

/* Static text for a status code, and the detail of the calling thread's last error. */
const char* ra_status_string(ra_status s);
const char* ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
