/*
 * abatt.h -- AB-Attention block-sparse video attention on MI355X (gfx950).
 *
 * C ABI of the library libabatt.so.  Three calls make the hot path:
 *
 *   abatt_plan    Q, K            -> CSR sampling plan (key-block ids + log-weights)
 *   abatt_attend  Q, K, V, plan   -> O (+ log-sum-exp)
 *   abatt_dense   Q, K, V         -> O (+ log-sum-exp), every key, no shift
 *
 * abatt_v_to_f16 + abatt_attend_v16 split abatt_attend in two (V converted to
 * fp16 once per call; the same results from a faster kernel);
 * abatt_plan_noalloc is abatt_plan without a caller workspace; test hooks
 * enter the same kernels part-way (abatt_key_means, abatt_scores,
 * abatt_plan_from_scores).
 *
 * Pages this follows:
 *   [hamidun]  news.hamidun.com, "AB-Attention speeds up video generation by
 *              up to 2.23x and skips 92% of attention"
 *   [zerohour] zerohour.day, "AB-Attention approximates dense video attention
 *              at high sparsity"
 *
 * Conventions shared by every call:
 *   - Q, K, V and O are [B, H, N, D] contiguous (row-major, D fastest), in
 *     the problem's dtype.  Tokens are in their original (raster) order: the
 *     library never permutes them ([hamidun] three techniques: the clustering
 *     only estimates importance; the computation runs in token order).
 *   - Q, K, V, O (and V16, kmean and workspaces) are read and written 16
 *     bytes at a time and must be 16-byte aligned, as every torch allocation
 *     is; a NULL or misaligned pointer is rejected with ABATT_EINVAL.
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates or frees device memory and never synchronises: each
 *     call checks its arguments on the host, enqueues kernels on `stream` and
 *     returns.  Scratch memory comes in through `workspace`.
 *   - The plan calls (abatt_plan, abatt_plan_onepass, abatt_plan_noalloc,
 *     abatt_scores) run their key-means kernel beside k-means on a second
 *     stream that the library creates once per device (default priority,
 *     kept until the process ends).  It is forked from `stream` by an event
 *     and joined back by another before the scorer, so the call's work stays
 *     ordered on `stream`.  While `stream` is under graph capture the side
 *     stream is not used (a stream that joins a capture stays in it until
 *     the capture ends, and would pull other threads' calls in): both
 *     kernels then run on `stream`, one after the other, with the same
 *     results.  abatt_plan_noalloc never creates the side stream.
 *   - Invalid arguments are reported synchronously, before any HIP call, as a
 *     negative abatt_status; nothing is enqueued then.  A failed launch gives
 *     ABATT_EHIP.  Device-side conditions (a plan that outgrew its capacity)
 *     are written to plan->status without a sync.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Apart from those side streams the library holds no state between
 *     calls, and it is thread-safe (a mutex orders the forks).  Calls on
 *     different streams need their own workspaces and plans.  The one
 *     exception is abatt_plan_noalloc, whose workspace is a static device
 *     array of the library shared by every call on a GPU (see there).
 *   - Query block qb holds tokens [q_block*qb, min(q_block*(qb+1), N)); key
 *     block j holds tokens [kv_block*j, kv_block*j + kv_block).  The last
 *     n_forced_tail tokens (text tokens) form "forced" key blocks that are not
 *     scored and are kept in every plan row with weight 1.
 *   - Plan row r belongs to (b, h, qb) with r = (b*H + h)*n_qb + qb,
 *     n_qb = ceil(N / q_block).
 *   - Inputs must be finite.  The attention kernels are built without IEEE
 *     NaN semantics (NaN-propagating max and compare are dropped from the
 *     softmax), and the selector's scores and sampler assume finite values:
 *     NaN or Inf anywhere in Q, K or V gives unspecified (but in-bounds)
 *     results.  Nothing checks this on the device.
 */
#ifndef ABATT_H
#define ABATT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABATT_OK = 0,
  ABATT_EINVAL = -1,        /* null pointer, bad size or bad parameter        */
  ABATT_EUNSUPPORTED = -2,  /* valid, but outside what the kernels implement */
  ABATT_EWORKSPACE = -3,    /* workspace smaller than *_workspace_bytes()     */
  ABATT_ECAPACITY = -4,     /* plan capacity below what the call may need     */
  ABATT_EHIP = -5,          /* a HIP launch failed                            */
  ABATT_ESCRATCH = -6       /* problem needs more than ABATT_SCRATCH_BYTES of */
                            /* plan workspace (abatt_plan_noalloc)            */
} abatt_status;

/* Size of the library's own device scratch array, which abatt_plan_noalloc
   uses as its plan workspace (256 MiB: the plan workspace of up to the
   12-head, 32760-token 480p layer, about 167 MB). */
#define ABATT_SCRATCH_BYTES (256u * 1024u * 1024u)

typedef enum { ABATT_F32 = 0, ABATT_BF16 = 1 } abatt_dtype;

typedef struct {
  int32_t B, H, N, D;       /* batch, heads, tokens, head dim; D in {64, 128}          */
  int32_t q_block;          /* query block size; the kernels implement 128             */
  int32_t kv_block;         /* key/value block size: 4 (the pages' choice) or another  */
                            /* power of two up to 128; dense attention ignores it     */
  int32_t n_clusters;       /* k-means clusters per query block: 8 or 16               */
  int32_t kmeans_iters;     /* Lloyd iterations, >= 1                                  */
  int32_t n_forced_tail;    /* trailing tokens kept in every row; multiple of kv_block */
  float scale;              /* logit scale, usually 1/sqrt(D); must be > 0             */
  abatt_dtype dtype;        /* dtype of Q, K, V and O                                  */
} abatt_problem_t;

typedef struct {
  int32_t *row_ptr;         /* [R+1] device: row r owns entries row_ptr[r]..row_ptr[r+1]-1   */
  int32_t *col_idx;         /* [capacity] device: key-block ids, ascending within a row      */
  float *logw;              /* [capacity] device: log(1/pi) >= 0 of each kept block          */
  int64_t capacity;         /* entries allocated in col_idx and logw                         */
  int32_t *status;          /* device int32 written by abatt_plan: 0 ok, 1 = the sampled     */
                            /* plan needs more than `capacity` entries (row_ptr then holds   */
                            /* the needed total in row_ptr[R]; col_idx/logw are not written  */
                            /* and abatt_attend treats every row as empty).  May be NULL for */
                            /* a plan filled by the caller.                                  */
} abatt_plan_t;

/* Number of plan rows R = B*H*ceil(N/q_block); -1 if *p is invalid. */
int64_t abatt_plan_rows(const abatt_problem_t *p);

/* Entries of a plan that keeps every block (budget 1): R * n_kb, where
   n_kb = (N - n_forced_tail)/kv_block + n_forced_tail/kv_block.  Always a
   safe capacity; -1 if *p is invalid. */
int64_t abatt_plan_max_nnz(const abatt_problem_t *p);

/* A capacity that a plan drawn at `budget` exceeds with negligible
   probability: per row min(n_kbs, ceil(m + 10*sqrt(m) + 16)) plus the forced
   blocks, m = budget*n_kbs (the row count is a sum of independent Bernoulli
   draws with mean m and variance <= m).  -1 if invalid. */
int64_t abatt_plan_nnz_bound(const abatt_problem_t *p, double budget);

/* Workspace bytes abatt_plan and abatt_scores need (block means, centroids,
   weights, the score matrix S [R, n_kbs] fp32, row counts).  0 if invalid. */
size_t abatt_plan_workspace_bytes(const abatt_problem_t *p);

/* Workspace bytes abatt_plan_from_scores needs (row counts).  0 if invalid. */
size_t abatt_sampler_workspace_bytes(const abatt_problem_t *p);

/*
 * abatt_plan -- IBCS selector followed by SIP sampling.
 *
 * [hamidun] "AB-Attention's three techniques", IBCS and SIP paragraphs, and
 * the third technique (4-token key blocks; kv_block may select another size):
 *   1. mean key of every sparse key block (kv_block consecutive tokens);
 *   2. per 128-query block, Lloyd k-means with n_clusters centroids (init at
 *      the evenly spaced members, kmeans_iters iterations); weight of a
 *      cluster = share of the block's queries in it;
 *   3. score s_j = sum_c w_c softmax_j(scale * mu_c . kmean_j) over the
 *      sparse key blocks, stored as fp32.  The dot products take fp16
 *      operands, scaled by powers of two so that any finite input keeps 11
 *      significant bits (bf16 problems), or bf16 hi + lo splits of both
 *      operands (fp32 problems); accumulation and softmax are fp32;
 *   4. inclusion probability pi_j proportional to s_j, capped at 1, summing
 *      to m = budget * n_kbs per row (float64 water-filling);
 *   5. block j kept iff word j%4 of Philox4x32-10(counter (j/4, qb, h, b),
 *      key (seed low, seed high)), a 32-bit uniform integer, is below
 *      pi_j * 2^32 (exact compare: inclusion probability within 2^-32 of
 *      pi_j);
 *   6. CSR rows in ascending block order, logw = log(1/pi) rounded to fp32
 *      (0 where pi = 1), forced blocks appended with logw 0.
 * budget in (0, 1]; budget 1 keeps every block.  Q, K: [B,H,N,D] device.
 * workspace: device, >= abatt_plan_workspace_bytes(p).  plan: host struct
 * whose pointers are device buffers; row_ptr [R+1]; capacity entries in
 * col_idx/logw (abatt_plan_nnz_bound() or abatt_plan_max_nnz()); status
 * non-NULL.  Returns ABATT_ECAPACITY synchronously if capacity is below
 * R * (number of forced blocks).
 */
abatt_status abatt_plan(const abatt_problem_t *p, const void *Q, const void *K,
                        double budget, uint64_t seed, void *workspace,
                        size_t workspace_bytes, abatt_plan_t *plan,
                        hipStream_t stream);

/*
 * abatt_plan_onepass -- abatt_plan with the sampler fused into one pass (the
 * fused-selector form that removes the second read of the score matrix).
 * Same arguments, checks, workspace and results, bit for bit, as
 * abatt_plan: the same scores, pi and draws.  One work-group per plan row,
 * rows taken in ticket order, solves pi, draws, finds the row's offset in
 * the plan from the counts of the rows before it (decoupled look-back over
 * one 64-bit record per row) and writes the row at once, so no scan or fill
 * launch follows and the score matrix comes from memory once.  On MI355X it
 * is slower than abatt_plan at 18 900 key blocks (1-4% of the plan: its one
 * kernel takes longer than count, scan and fill together) and about equal at
 * 29 700; it is kept for that comparison.
 *   - The look-back waits only for rows that took their tickets earlier, so
 *     it always ends; its spin is bounded all the same, and a plan whose
 *     look-back hit the bound gets *status = 2 (invalid, like an overflow).
 *   - On overflow (*status = 1) the rows that fit may have been written;
 *     the plan is invalid as with abatt_plan.
 *   - Concurrent calls need separate workspaces, as for abatt_plan.
 */
abatt_status abatt_plan_onepass(const abatt_problem_t *p, const void *Q, const void *K,
                                double budget, uint64_t seed, void *workspace,
                                size_t workspace_bytes, abatt_plan_t *plan,
                                hipStream_t stream);

/*
 * abatt_plan_noalloc -- abatt_plan for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, checks and results (bit for bit) as
 * abatt_plan, without the workspace: the plan workspace lives in a static
 * device array of ABATT_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends.
 * The call itself allocates and frees nothing and creates no stream (it
 * forks onto a side stream only when an earlier plan call on the GPU made
 * one); the caller still provides Q, K and the plan buffers.
 *   - Returns ABATT_ESCRATCH, before any HIP call, when
 *     abatt_plan_workspace_bytes(p) > ABATT_SCRATCH_BYTES (call it per group
 *     of heads instead: the plan rows of a head depend on that head only).
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents (every kernel writes its part before reading it,
 *     so nothing has to be cleared).  Calls that overlap on one GPU -- on
 *     different streams, or from different threads without ordering -- race
 *     on the array and give undefined plans: serialise them.
 *   - The device address of the array is looked up on the first call on
 *     each device (hipGetSymbolAddress, with that device current);
 *     ABATT_EHIP if that fails.
 */
abatt_status abatt_plan_noalloc(const abatt_problem_t *p, const void *Q, const void *K,
                                double budget, uint64_t seed, abatt_plan_t *plan,
                                hipStream_t stream);

/*
 * abatt_attend -- softmax attention over the plan's gathered key blocks.
 *
 * [hamidun] three techniques, SIP: ordinary softmax attention whose logits
 * get the shift log(1/pi) of their block (Horvitz-Thompson weighting), and
 * third technique / [zerohour] key facts: the kept 4-token K/V blocks
 * (kv_block tokens in general) are gathered by index into full compute
 * tiles, tokens are not permuted.
 * For query i of row r and kept token t of block j(t):
 *   z_t = scale * q_i . k_t + logw_j(t);  o_i = sum_t e^(z_t - M) v_t / l,
 *   l = sum_t e^(z_t - M);  lse_i = M + ln l  (natural log).
 * A row with no kept block gives o = 0 and lse = -inf.  Block ids outside
 * [0, n_kb) are skipped.  O: [B,H,N,D] device, written in full.  lse: NULL or
 * [B,H,N] fp32 device.  bf16 path: QK^T on bf16 MFMA with fp32 accumulation,
 * fp32 softmax, PV on fp16 MFMA (probabilities and the bf16 values converted
 * to fp16), O rounded to bf16.  f32 path: fp32 arithmetic throughout.
 */
abatt_status abatt_attend(const abatt_problem_t *p, const void *Q, const void *K,
                          const void *V, const abatt_plan_t *plan, void *O,
                          float *lse, hipStream_t stream);

/*
 * abatt_v_to_f16, abatt_attend_v16 -- abatt_attend in two steps, for bf16
 * problems ([hamidun] three techniques: the same gathered attention).
 *
 * The bf16 path multiplies the probabilities with V in fp16.  abatt_attend
 * converts each gathered V block while staging it, once for every plan row
 * that keeps the block.  abatt_v_to_f16 converts V once per call instead:
 * V16[i] = V[i] rounded toward zero to fp16, with the same instruction
 * abatt_attend uses.  That is exact for |v| in fp16's normal range
 * [2^-14, 65504]; larger magnitudes saturate and smaller ones lose bits.
 * abatt_attend_v16 then takes V16 in place of V and moves it to LDS by
 * direct loads, like K.  Its O and lse are bit-identical to abatt_attend's
 * on the V that V16 came from.
 *
 * V, V16: [B,H,N,D] device buffers of 2-byte elements, caller-owned; V16 is
 * written in full and must not be V.  abatt_v_to_f16 checks the problem as
 * abatt_dense does (any N; kv_block and n_forced_tail are not used).  Other arguments as abatt_attend.
 * Returns ABATT_EUNSUPPORTED for fp32 problems, and ABATT_EINVAL for NULL
 * pointers or V16 == V.
 */
abatt_status abatt_v_to_f16(const abatt_problem_t *p, const void *V, void *V16,
                            hipStream_t stream);
abatt_status abatt_attend_v16(const abatt_problem_t *p, const void *Q, const void *K,
                              const void *V16, const abatt_plan_t *plan, void *O,
                              float *lse, hipStream_t stream);

/*
 * abatt_dense -- full softmax attention over every key, no shift: the
 * quadratic baseline the method approximates ([hamidun] introduction;
 * [zerohour] abstract excerpt).  Same layouts, precision and lse convention
 * as abatt_attend.
 */
abatt_status abatt_dense(const abatt_problem_t *p, const void *Q, const void *K,
                         const void *V, void *O, float *lse, hipStream_t stream);

/*
 * abatt_dense_v16 -- abatt_dense with V given as fp16 (from abatt_v_to_f16),
 * for bf16 problems: the dense kernel then stages V as it is instead of
 * converting each chunk for every query block.  O and lse are bit-identical to
 * abatt_dense's on the V that V16 came from.  Same checks as abatt_dense;
 * ABATT_EUNSUPPORTED for fp32 problems.
 */
abatt_status abatt_dense_v16(const abatt_problem_t *p, const void *Q, const void *K,
                             const void *V16, void *O, float *lse, hipStream_t stream);

/*
 * Test hooks: the selector's kernels entered part-way.
 *
 * abatt_key_means: kmean [B,H,n_kbs,D] fp32 device = mean of each sparse
 * key block of kv_block tokens ([hamidun] three techniques, IBCS: averaged
 * keys).
 *
 * abatt_scores: steps 1-3 of abatt_plan.  S [R, n_kbs] fp32 device;
 * centroids [R, n_clusters, D] fp32 device and weights [R, n_clusters] fp32
 * device (either may be NULL).  workspace as for abatt_plan.
 *
 * abatt_plan_from_scores: steps 4-6 of abatt_plan from caller scores
 * S [R, n_kbs] fp32 device (non-negative).  workspace >=
 * abatt_sampler_workspace_bytes(p).
 */
abatt_status abatt_key_means(const abatt_problem_t *p, const void *K, float *kmean,
                             hipStream_t stream);
abatt_status abatt_scores(const abatt_problem_t *p, const void *Q, const void *K,
                          float *S, float *centroids, float *weights,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);
abatt_status abatt_plan_from_scores(const abatt_problem_t *p, const float *S,
                                    double budget, uint64_t seed, void *workspace,
                                    size_t workspace_bytes, abatt_plan_t *plan,
                                    hipStream_t stream);

/* Static description of a status code. */
const char *abatt_status_str(abatt_status s);

/* Library version string. */
const char *abatt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ABATT_H */
