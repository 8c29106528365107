/*
 * prr.h — C ABI of libprr: one decode step of PRR's dynamic sparse attention for one attention layer on one
 * MI355X (gfx950).
 *
 * Method: "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM Decoding"
 * (arXiv 2606.30389). PRR abstract: decoding attends to the top-K KV blocks of each query; an EMA-based predictor
 * forecasts those blocks, attention is speculated over them while the true selection is in flight, and once the
 * true set is known the missed blocks are folded into the partial attention state with online-softmax statistics.
 * PRR summary page (Key findings, Contributions): the repair covers exactly the missed blocks, so the result equals
 * standard DSA over the true top-K set.
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers to contiguous row-major buffers that the caller allocates, owns and
 *    frees. The library never allocates device memory, never synchronises the host, and launches only on the
 *    stream(s) it is given (a hipStream_t passed as void*; NULL = the null stream).
 *  - Calls are asynchronous: they validate their arguments on the host, enqueue kernels and return. A non-zero
 *    status means nothing was enqueued (PRR_EINVAL, PRR_EUNSUPPORTED) or a launch failed (PRR_ELAUNCH);
 *    prr_last_error() then gives a thread-local message. Device faults surface at the caller's next sync.
 *  - Inputs must be finite (no NaN/Inf in q, K, V).
 *  - No state lives in the library: the EMA vector, index lists and partials are caller buffers, so any number of
 *    layers (each with its own buffers) may share the library.
 *
 * Notation: B batch, Hq query heads, Hkv KV heads, G = Hq / Hkv (query head h uses KV head h / G), D head_dim,
 * bs block_size (tokens per selection block), N n_blocks = ctx / bs, K top_k, K' k_spec (speculation budget).
 * The storage dtype (prr_dtype) applies to q, the K/V caches and the summaries; all scores, EMA values, partials
 * and outputs are fp32.
 *
 * Layouts
 *  q          [B, Hq, D]
 *  k/v cache  [n_pages, Hkv, page_size, D]   (PagedAttention, PRR reference list); token i of sequence b lives in
 *             physical page block_table[b, i / page_size], row i % page_size
 *  block_table int32 [B, pages_per_seq], pages_per_seq = N * bs / page_size
 *  summaries  [B, Hkv, N, 2, D]   row 0 = elementwise min of the block's keys, row 1 = max (Quest)
 *  scores     f32 [B, Hkv, N]
 *  ema        f32 [B, Hkv, N]
 *  sel_idx    int32 [B, Hkv, K]   ascending block ids of the true top-K set
 *  pred_idx   int32 [B, Hkv, K']  ascending block ids of the predicted set
 *  partials   buffer of prr_partials_bytes() (passed as float*): one record per (b, kv head, predicted slot),
 *             layout [B, Hkv, K'] x {m[G], l[G] fp32, zero padding to a multiple of 4 floats, O[G][D]}; m is the
 *             block's largest logit in log2 units (softmax_scale * q.k * log2 e), l = sum of 2^(z - m), O = sum of
 *             2^(z - m) v (unnormalised); O is stored in fp32 for fp32 storage, and as O / l (the block's own
 *             attention output, a weighted average of its values) in fp16, rounded to nearest even, for bf16 and
 *             fp16 storage (values beyond the fp16 range, |v| > 65504 in a bf16 cache, are not supported there);
 *             records are 16-byte aligned
 *  out        f32 [B, Hq, D]      softmax attention over the tokens of the true top-K blocks
 *  n_missed   int32 [B, Hkv]      |T \ P| of the last repair
 */
#ifndef PRR_H_
#define PRR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRR_OK = 0,
  PRR_EINVAL = -1,        /* a null pointer, a size out of range or inconsistent shapes */
  PRR_EUNSUPPORTED = -2,  /* a valid but unsupported combination (dtype x head_dim, group size) */
  PRR_ELAUNCH = -3        /* the HIP runtime reported an error when enqueuing */
} prr_status;

typedef enum { PRR_F32 = 0, PRR_BF16 = 1, PRR_F16 = 2 } prr_dtype;

/* Block scorer. QUEST: the summary slot of a block holds its elementwise key min and max (2 rows of D elements of the
 * cache dtype) and the score is Quest's bound (PRR reference list, Quest). MEAN: the same 2 * D * elem-size bytes hold
 * the block's mean key in fp32 (D floats; with fp32 storage the second half of the slot is unused) and the score is
 * the group-summed query against it — a representative-key scorer (the PRR abstract evaluates representative DSA
 * methods). */
typedef enum { PRR_SCORER_QUEST = 0, PRR_SCORER_MEAN = 1 } prr_scorer;

/* Shape of one attention layer's decode state. Supported: (dtype F32, head_dim 64) and (dtype BF16 or F16,
 * head_dim 128) — one 256-byte row per token; group size G in {1, 2, 4, 8}; block_size a multiple of page_size and
 * of 4; 1 <= n_blocks <= 65536 (and n_blocks <= 32768 for the top-K kernels).
 * ctx_len: tokens of every sequence. 0 means n_blocks * block_size; otherwise (n_blocks - 1) * block_size < ctx_len
 * <= n_blocks * block_size, and the last block holds ctx_len - (n_blocks - 1) * block_size tokens: its summary covers
 * those tokens and attention never reads past them (decode appends one token at a time, prr_append_kv). */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t block_size, page_size;
  int32_t n_blocks, pages_per_seq;
  int32_t dtype;        /* prr_dtype */
  float softmax_scale;  /* typically 1/sqrt(head_dim) */
  int32_t ctx_len;      /* tokens per sequence (0: n_blocks * block_size) */
  int32_t sink_blocks;  /* forced blocks: the first sink_blocks and the last local_blocks of every sequence rank   */
  int32_t local_blocks; /* above all others in every top-K (true set and prediction), among themselves by index; */
                        /* sink_blocks + local_blocks <= n_blocks (0, 0: plain top-K)                            */
  int32_t scorer;       /* prr_scorer                                                                            */
} prr_shape;

/* Quest block summaries (PRR reference list, Quest): for every (b, kv head g, block n), the elementwise min and max
 * over the block's tokens of the keys, read through the page table; exact in every dtype. With the MEAN scorer the
 * slot receives the block's mean key in fp32 instead (summed in fp32, divided by the block's token count).
 * block_ids: NULL rebuilds every block; otherwise n_block_ids flat ids f = (b * Hkv + g) * N + n (e.g. the blocks
 * whose keys changed) are rebuilt and the rest of `summaries` is left untouched. */
prr_status prr_build_summaries(const prr_shape* shape, const void* k_cache, const int32_t* block_table,
                               const int32_t* block_ids, int32_t n_block_ids, void* summaries, void* stream);

/* Decode-time append (the step before selection in a decoder): with ctx_len the length after the append, the token
 * at position p = ctx_len - 1 of every (b, kv head g) is written from k_new, v_new [B, Hkv, D] (the cache dtype) into
 * the K and V caches through the block table, and the summary of its block n = p / block_size is updated in place:
 * (k, k) when p starts the block, else the elementwise (min, max) with k — exact, and equal to rebuilding the
 * block's summary over its tokens. Requires ctx_len >= 1 (a shape with ctx_len 0 appends at n_blocks * block_size - 1,
 * the last slot). Enqueues one small launch; the next step's shape carries the same ctx_len. */
prr_status prr_append_kv(const prr_shape* shape, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* block_table, void* summaries, void* stream);

/* Query-aware block scores and exact top-K selection (PRR abstract: attend only to the top-K blocks relevant to
 * each query). scores[b,g,n] = sum over the query heads h of KV head g and dims d of
 * max(q[b,h,d]*kmin[d], q[b,h,d]*kmax[d]) (fp32); sel_idx[b,g,:] = the top_k largest scores, ties to the lower
 * block index, ascending. Requires 1 <= top_k <= N. `workspace` (prr_workspace_bytes bytes, no initialisation
 * needed) or NULL: with it, rows of more than 8192 blocks select in two launches (the top-K of each segment of 4096
 * scores, then the top-K of those candidates), much faster on long rows than one workgroup per row; the result is
 * the same. The selection uses the workspace's true-set candidate region only. */
prr_status prr_score_select(const prr_shape* shape, const void* q, const void* summaries, int32_t top_k,
                            float* scores, int32_t* sel_idx, void* workspace, void* stream);

/* Per-row budgets of the predicted set (PRR summary page: speculative work is held to a dynamic budget; its future
 * work: adaptive budgeting, and confidence measures for the EMA predictor). The pages give no formula; these two
 * rules are readings. With a budget, row r of a predicted set holds k_r <= k_spec ascending block ids followed by
 * k_spec - k_r entries of -1 (empty slots, which speculation skips and repair never matches):
 *   PRR_BUDGET_MISSES:     k_r = K + ceil(beta * m_r), m_r = missed_prev[r], the blocks row r missed at its last
 *                          completed step (fp32 product), clamped to [k_min, k_spec]; the set is the top-k_r of the
 *                          EMA (forced blocks first).
 *   PRR_BUDGET_CONFIDENCE: with u_n = e_n + c * |s_n - e_n| (fp32; e the updated EMA, s the step's scores), k_r is
 *                          the number of blocks whose u reaches the K-th entry of the EMA in the selection order
 *                          (forced blocks first; a forced block reaches every value, and when the K-th entry is
 *                          forced only forced blocks reach it), clamped to [k_min, k_spec]; the set is the top-k_r
 *                          of u (forced blocks first, ties to the lower index).
 * K = top_k, the decode step's true-set size. A NULL budget, or policy PRR_BUDGET_FIXED, keeps k_r = k_spec. */
typedef enum { PRR_BUDGET_FIXED = 0, PRR_BUDGET_MISSES = 1, PRR_BUDGET_CONFIDENCE = 2 } prr_budget_policy;
typedef struct {
  int32_t policy;               /* prr_budget_policy                                                              */
  int32_t top_k;                /* K, 1 <= top_k <= N                                                             */
  int32_t k_min;                /* 1 <= k_min <= k_spec                                                           */
  float beta;                   /* PRR_BUDGET_MISSES: blocks added per missed block, finite, >= 0                */
  float c;                      /* PRR_BUDGET_CONFIDENCE: weight of |s - e|, finite, >= 0                         */
  const int32_t* missed_prev;   /* PRR_BUDGET_MISSES: int32 [B, Hkv] on the device (a buffer the step did not
                                   just write: double-buffer the missed counts across steps)                      */
} prr_budget;

/* EMA score predictor (PRR abstract: a light predictor built on an exponential moving average): ema = scores when
 * first_step != 0, else ema = alpha * ema + (1 - alpha) * scores (in place); then pred_idx_next[b,g,:] = top-k_spec
 * of ema, ties to the lower index, forced blocks first (as the selection), ascending — the predicted set for the next
 * decode step. Requires 1 <= k_spec <= N. `workspace` as in prr_score_select (its predicted-set candidate region
 * only, so the two selections may run at once). `budget` (NULL: fixed) sizes each row's set as described above; a
 * budgeted row selects in one workgroup (rows of at most 32768 blocks) and does not use the workspace. */
prr_status prr_ema_predict(const prr_shape* shape, const float* scores, float* ema, float alpha, int32_t first_step,
                           int32_t k_spec, int32_t* pred_idx_next, const prr_budget* budget, void* workspace,
                           void* stream);

/* Speculative attention (PRR abstract: speculate the attention over the predicted blocks while selection is in
 * flight): for every (b, g) and predicted slot j < k_spec, with n = pred_idx[b,g,j] and each query head h of the
 * group, z_i = softmax_scale * q[b,h] . k_i over the block's tokens; the block's partial state m = max z,
 * l = sum exp(z - m), O = sum exp(z - m) v_i is stored as the record (b, g, j) of `partials`, in the base-2 form
 * given under Layouts (m2 = m * log2 e, the same l and O). k_spec == 0 enqueues nothing. A negative id marks an
 * empty slot (a budgeted prediction's padding): nothing is computed or written for it; empty slots must follow every
 * id of their row. Ids >= N are clamped to N - 1 (a wrong result, never an out-of-bounds read). */
prr_status prr_speculate(const prr_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* pred_idx, int32_t k_spec, float* partials,
                         void* stream);

/* Repair and merge (PRR abstract: repair the missed blocks once the true set is known; folds them into the partial
 * state with online-softmax statistics). For every (b, g): the blocks of T = sel_idx[b,g,:] that are in
 * P = pred_idx[b,g,:k_spec] reuse their speculated partials; the missed blocks M = T \ P are computed here; blocks of
 * P \ T never enter. P ends at its first negative (empty) slot: ids after it are never matched, so a block of T
 * listed there is computed as missed. out[b,h] = O / l of the merged state; n_missed[b,g] = |M|. k_spec == 0 (or pred_idx NULL)
 * computes attention over all of T (the serialized select-then-attend path). `workspace` holds
 * prr_workspace_bytes() bytes of scratch (no initialisation needed); it uses the workspace's repair region, so it
 * may overlap a selection call on the same workspace, but not another repair. */
prr_status prr_repair_merge(const prr_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* sel_idx, int32_t top_k,
                            const int32_t* pred_idx, int32_t k_spec, const float* partials, float* out,
                            int32_t* n_missed, void* workspace, void* stream);

/* Block scores alone (as in prr_score_select) and, when ema != NULL, the EMA update of prr_ema_predict in the same
 * pass over the summaries (ema = scores when first_step != 0, else alpha * ema + (1 - alpha) * scores, in place). The
 * first half of the fused single-stream step; prr_select_speculate is the second. */
prr_status prr_score(const prr_shape* shape, const void* q, const void* summaries, float* scores, float* ema,
                     float alpha, int32_t first_step, void* stream);

/* In ONE launch: the true top-K of `scores` into sel_idx (as prr_score_select); when k_spec_next > 0 the next
 * step's predicted set pred_idx_next = top-k_spec_next of `ema` (already updated by prr_score; ties to the lower
 * index, ascending); and the speculation of prr_speculate over pred_idx (k_spec slots) into `partials`.
 * Selection occupies one workgroup per row and is bound by latency, so speculation runs in its shadow (PRR
 * abstract: speculation overlaps selection). pred_idx and pred_idx_next must be different buffers. `workspace`
 * (prr_workspace_bytes bytes) or NULL: with it, rows of more than 8192 blocks (with top_k and k_spec_next <= 1024)
 * select by segments of 2048 values in this launch and merge the candidates in a second one. `budget` (NULL: fixed)
 * sizes each row of pred_idx_next as in prr_ema_predict (`scores` are the step's s, `ema` the updated e); with the
 * workspace, budgeted long rows select by segments too (a confidence budget uses the third candidate region). */
prr_status prr_select_speculate(const prr_shape* shape, const float* scores, int32_t top_k, int32_t* sel_idx,
                                const float* ema, int32_t k_spec_next, int32_t* pred_idx_next, const void* q,
                                const void* k_cache, const void* v_cache, const int32_t* block_table,
                                const int32_t* pred_idx, int32_t k_spec, float* partials, const prr_budget* budget,
                                void* workspace, void* stream);

/* Scores (+ the EMA update when ema != NULL, as prr_score) and the speculation of prr_speculate over pred_idx
 * (k_spec slots), in ONE launch whose workgroups of the two roles run concurrently (PRR abstract: speculation runs
 * while selection is in flight). The first half of the two-launch step; prr_select_repair is the second. */
prr_status prr_score_speculate(const prr_shape* shape, const void* q, const void* summaries, float* scores, float* ema,
                               float alpha, int32_t first_step, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* pred_idx, int32_t k_spec, float* partials,
                               void* stream);

/* Selection with repair (PRR abstract: repair the missed blocks once the true set is known), in two launches. Per
 * (b, g) row: the true top-K of `scores` into sel_idx (as prr_score_select); then, in the same workgroup, the blocks
 * of T missing from P = pred_idx[b,g,:k_spec] are attended from the KV cache and merged into one partial state;
 * a second launch merges that state with the records of the blocks of T ∩ P found in `partials` (written before by
 * prr_score_speculate or prr_speculate) — blocks of P outside T never enter — and writes out = O / l and
 * n_missed = |T minus P| as prr_repair_merge does. When k_spec_next > 0 other workgroups of the first launch also
 * write pred_idx_next = top-k_spec_next of `ema` (already updated). k_spec == 0 attends over all of T
 * (select-then-attend). `workspace` holds prr_workspace_bytes(shape, top_k) bytes (no initialisation needed; it uses
 * the repair region, as prr_repair_merge). Returns PRR_EUNSUPPORTED unless page_size is a multiple of 16,
 * block_size <= 128 and top_k, k_spec, k_spec_next <= 2048 (the separate calls cover the rest). pred_idx is searched
 * by bisection when ascending (as the top-K calls write it), linearly otherwise. */
prr_status prr_select_repair(const prr_shape* shape, const float* scores, int32_t top_k, int32_t* sel_idx,
                             const float* ema, int32_t k_spec_next, int32_t* pred_idx_next, const void* q,
                             const void* k_cache, const void* v_cache, const int32_t* block_table,
                             const int32_t* pred_idx, int32_t k_spec, const float* partials, float* out,
                             int32_t* n_missed, void* workspace, void* stream);

/* Bytes of the partials buffer for a speculation budget k_spec (0 for k_spec == 0). */
size_t prr_partials_bytes(const prr_shape* shape, int32_t k_spec);
/* Bytes of the workspace of the selection calls, prr_repair_merge, prr_select_repair and prr_decode_step for top_k:
 * three top-K candidate regions (true set, predicted set, a confidence budget's optimistic scores; empty unless
 * N > 8192), then the repair region. */
size_t prr_workspace_bytes(const prr_shape* shape, int32_t top_k);

/* ---- one decode step on two streams (the runtime around the calls above) ------------------------------------ */

typedef enum {
  PRR_MODE_SERIALIZED = 0,  /* stream_sel: score_select -> repair_merge over all of T (no prediction)            */
  PRR_MODE_ONE_STREAM = 1,  /* stream_sel: speculate -> score_select -> repair_merge -> ema_predict                */
  PRR_MODE_TWO_STREAM = 2,  /* stream_spec: speculate || stream_sel: score_select; after the join, repair_merge
                               -> ema_predict on stream_sel (one fork and one join per step)                    */
  PRR_MODE_FUSED = 3,       /* stream_sel only. batch * n_kv_heads >= 128: speculate -> score -> one launch of
                               top-K workgroups selecting T and P_{t+1}, the latter updating the EMA first
                               (rows of more than 8192 blocks by segments and a merge) -> repair_merge (the
                               hits' records merged, the missed blocks attended). Otherwise, top_k <= 32:
                               score -> one launch selecting T and P_{t+1} (after the EMA update), speculating
                               over P_t and attending T minus P_t per row -> merge. Otherwise: score ->
                               select_speculate (T, P_{t+1} after the EMA update, speculation over P_t; rows of
                               more than 8192 blocks by segments and a merge) -> repair_merge, which with nothing
                               to speculate or predict are the serialized launches. Under a per-row budget below
                               128 rows the scoring pass updates the EMA. The shapes each form supports are
                               the conditions of the separate calls; outside them the next form is taken.      */
  PRR_MODE_SERIALIZED_FUSED = 4  /* stream_sel only: score -> select_repair with no prediction (select-then-attend
                                    in two launches) when select_repair supports the shape and batch * n_kv_heads
                                    >= 128; otherwise as PRR_MODE_SERIALIZED                                    */
} prr_mode;

typedef struct {
  const void* q; const void* k_cache; const void* v_cache; const int32_t* block_table; const void* summaries;
  float* scores;               /* written by score_select, read by ema_predict; double-buffer it across steps   */
  int32_t* sel_idx;
  float* ema;
  const int32_t* pred_cur;     /* P_t (k_spec_cur entries; ignored when k_spec_cur == 0)                          */
  int32_t* pred_next;          /* P_{t+1} (k_spec_next entries), written by ema_predict                          */
  float* partials;             /* speculation partials for P_t; double-buffer it across steps                   */
  float* out; int32_t* n_missed; void* workspace;
  int32_t top_k, k_spec_cur, k_spec_next, first_step;
  float alpha;
  const prr_budget* budget;    /* NULL: fixed k_spec_next per row; else per-row budgets (prr_ema_predict). pred_cur
                                  may then hold empty (-1) slots. Its top_k must equal this step's top_k. */
} prr_step_args;

/* Opaque host object holding the events that order the two streams (no device memory). */
typedef struct prr_step_ctx prr_step_ctx;
prr_status prr_step_ctx_create(prr_step_ctx** out);
void prr_step_ctx_destroy(prr_step_ctx* ctx);
/* Race check of the two-stream step: every later PRR_MODE_TWO_STREAM step with this context enqueues a bounded sleep
 * kernel of delay_spec iterations on stream_spec before the speculation and one of delay_sel iterations on
 * stream_sel between the join and the repair (one iteration is about 8000 shader clocks; 0 = none; each in
 * [0, 100000]). The results must not change: a step whose streams were wrongly ordered would read partial records
 * or predicted sets that are not yet written, or that the other stream overwrites. Test instrumentation. */
prr_status prr_step_ctx_set_delays(prr_step_ctx* ctx, int32_t delay_sel, int32_t delay_spec);

/* Enqueue one PRR decode step. Two-stream order (PRR abstract: speculation runs while selection is in flight), one
 * fork and one join per step:
 *   stream_sel:  [record fork] score_select [wait join] repair_merge ema_predict -> P_{t+1}
 *   stream_spec: [wait fork] speculate(P_t) [record join]
 * `out` and P_{t+1} are complete on stream_sel when the call's work there finishes; the next call's speculation is
 * ordered after them by its fork. stream_spec's work always ends in the join, so a graph capture of steps on
 * stream_sel is closed; `join` is accepted and has no further effect. In PRR_MODE_ONE_STREAM and PRR_MODE_SERIALIZED
 * only stream_sel is used. */
prr_status prr_decode_step(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* args, int32_t mode,
                           int32_t join, void* stream_sel, void* stream_spec);

/* ---- the same step without a caller workspace ---------------------------------------------------------------- */

/* Bytes of the library's static scratch that prr_decode_step_noalloc uses as its workspace. */
#define PRR_SCRATCH_MAX_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): prr_decode_step with the workspace taken from a file-scope device array of
 * PRR_SCRATCH_MAX_BYTES bytes that the library holds on every GPU it runs on until the process ends. args->workspace
 * must be NULL; every other argument, mode and result is as in prr_decode_step (same kernels, same order, so the
 * same bits). Calls nothing that allocates. Returns PRR_EINVAL when prr_workspace_bytes(shape, args->top_k) exceeds
 * PRR_SCRATCH_MAX_BYTES, or when a stream is not on the current device; PRR_ELAUNCH when the scratch's device address
 * cannot be taken (first call on a device). All calls on one GPU share its scratch, which keeps the last call's
 * contents (the workspace needs no initialisation): calls that overlap on one GPU (two streams, two threads, two
 * layers in flight) race; order them. */
prr_status prr_decode_step_noalloc(prr_step_ctx* ctx, const prr_shape* shape, const prr_step_args* args,
                                   int32_t mode, int32_t join, void* stream_sel, void* stream_spec);

/* Profiling-guided speculation budget (PRR abstract; PRR summary page, Limitations: polynomial regression outside
 * the profiled grid). Returns the largest kspec_grid[i] with t_spec[i] <= t_sel(n_target), where t_sel(n_target)
 * is t_sel[j] if n_grid[j] == n_target, else a least-squares polynomial of degree poly_degree (clamped to
 * n_pts_sel - 1, at most 4) fitted to (n_grid, t_sel). Returns 0 when no positive budget qualifies and -1 on
 * invalid arguments (null arrays, n_pts_sel < 1). Host-only; safe without a GPU. */
int32_t prr_choose_budget(const double* n_grid, const double* t_sel, int32_t n_pts_sel, const double* kspec_grid,
                          const double* t_spec, int32_t n_pts_spec, double n_target, int32_t poly_degree);

/* Profiling-guided budget of the fused single-stream step (PRR_MODE_FUSED). There the speculation shares the
 * selection launch, so its cost (a longer launch) and its saving (fewer missed blocks to repair) show only in the
 * step's own time: t_step[i] is the measured time of a decode step at budget kspec_grid[i], the grid holding 0 (the
 * step without speculation). Returns the largest kspec_grid[i] with t_step[i] <= the time at 0, i.e. the largest
 * budget that keeps speculation off the step's critical path; -1 on invalid arguments (null arrays, n_pts < 1, no
 * zero entry, a negative budget or a non-finite time). Host-only; safe without a GPU. */
int32_t prr_choose_budget_fused(const double* kspec_grid, const double* t_step, int32_t n_pts);

/* ---- kernel tracing ------------------------------------------------------------------------------------------ */
/* Per-kernel launch timing with HIP events recorded on the stream each kernel is launched on, for measuring the
 * achieved bandwidth of one kernel inside a running decode loop. A trace holds `capacity` event pairs per kernel
 * id; while enabled (process-wide, one trace at a time) every launch of a kernel in `kernel_mask` (bit i = kernel
 * id i) records an event immediately before and after it, until that kernel's pool is full. Reading synchronises
 * on the events. Under stream capture the records become external event nodes of the graph (each replay records
 * them again), so a captured decode loop can be traced too; such a graph refers to the trace's events, so destroy
 * every graph captured while a trace was enabled before destroying that trace. */
typedef enum {
  PRR_KERNEL_SUMMARIES = 0, PRR_KERNEL_SCORE = 1, PRR_KERNEL_SELECT_TOPK = 2, PRR_KERNEL_EMA_TOPK = 3,
  PRR_KERNEL_SPECULATE = 4, PRR_KERNEL_REPAIR = 5, PRR_KERNEL_FINALIZE = 6, PRR_KERNEL_COUNT = 7
} prr_kernel_id;
typedef struct prr_trace prr_trace;
prr_status prr_trace_create(prr_trace** out, int32_t capacity);
void prr_trace_destroy(prr_trace* trace);
/* Enable `trace` for the kernels in kernel_mask (0 or a NULL trace disables tracing); resets its counters. */
prr_status prr_trace_enable(prr_trace* trace, uint32_t kernel_mask);
/* Copy up to `cap` per-launch durations (ms) of `kernel` into ms_out; returns the count (>= 0) or a negative
 * prr_status. Synchronises on the recorded events. */
int32_t prr_trace_read(prr_trace* trace, int32_t kernel, float* ms_out, int32_t cap);

/* ---- benchmark helpers ----------------------------------------------------------------------------------- */
/* Write `bytes` (multiple of 16) of `buf` with a streaming kernel (evicts caches before cold-cache timing). */
prr_status prr_flush_write(void* buf, size_t bytes, void* stream);
/* Stream-read `bytes` (multiple of 16) of `buf`, writing one float per workgroup to `sink` (>= 65536 floats);
 * measures the achievable read bandwidth. */
prr_status prr_stream_read(const void* buf, size_t bytes, float* sink, void* stream);

const char* prr_status_string(prr_status s);
const char* prr_last_error(void);
/* Library version string. */
const char* prr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PRR_H_ */
