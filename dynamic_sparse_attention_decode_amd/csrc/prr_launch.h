// prr_launch.h — host-side declarations shared by the kernel translation units and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prr.h"

namespace prr {

// Thread-local error message for prr_last_error().
void set_error(const char* fmt, ...);
// Checks hipGetLastError() after a launch; on failure records the message and returns PRR_ELAUNCH.
prr_status check_launch(const char* what);

// Record of a partial attention state for one (b, g, slot): m[G] (log2 units), l[G], padding to a multiple of 4
// floats, then O[G][D]. Records are 16-byte aligned.
__host__ __device__ constexpr int rec_ml(int G) { return (2 * G + 3) & ~3; }
__host__ __device__ constexpr int64_t rec_floats(int G, int D) { return (int64_t)rec_ml(G) + (int64_t)G * D; }
// A speculation record (the partials buffer): m[G] and l[G] in fp32, zero padding to a multiple of 4 floats, then
// O[G][D]: for fp32 storage (dt 0) O itself in fp32; for 16-bit storage (dt 1, 2) O / l (the block's attention
// output, a weighted average of its values) in fp16, which the reader multiplies back by l. 16-byte aligned. Records
// inside the workspace keep O in fp32.
__host__ __device__ constexpr int spec_o_bytes(int dt) { return dt == 0 ? 4 : 2; }
__host__ __device__ constexpr int64_t spec_rec_bytes(int dt, int G, int D) {
  return (int64_t)rec_ml(G) * 4 + (int64_t)G * D * spec_o_bytes(dt);
}
// Four consecutive O values (dims 4 * slot .. 4 * slot + 3 of head h) of a record: an fp32 record's O when f32, else
// a compact speculation record's fp16 O / l times its l.
template <int G, int D>
__device__ inline float4 rec_o4(const uint8_t* __restrict__ rec, bool f32, int h, int slot) {
  constexpr int MLB = rec_ml(G) * 4;
  const int64_t e = (int64_t)h * D + slot * 4;
  if (f32) return *reinterpret_cast<const float4*>(rec + MLB + e * 4);
  const float l = reinterpret_cast<const float*>(rec)[G + h];
  const float4 v = unpack_f16x4(*reinterpret_cast<const uint2*>(rec + MLB + e * 2));
  return make_float4(v.x * l, v.y * l, v.z * l, v.w * l);
}

// Kernel tracing hooks: record the armed trace's start/end events around a launch of kernel `kid` on `stream`.
void trace_begin(int kid, hipStream_t stream);
void trace_end(int kid, hipStream_t stream);

// Calls FN<dtype, G>(args...) for the shape's storage dtype and group size (shape variable `s`).
#define PRR_DISPATCH_DT_G(FN, ...)                                      \
  do {                                                                  \
    const int G_ = s.n_q_heads / s.n_kv_heads;                          \
    if (s.dtype == 0) {                                              \
      switch (G_) {                                                     \
        case 1: FN<0, 1>(__VA_ARGS__); break;                        \
        case 2: FN<0, 2>(__VA_ARGS__); break;                        \
        case 4: FN<0, 4>(__VA_ARGS__); break;                        \
        default: FN<0, 8>(__VA_ARGS__); break;                       \
      }                                                                 \
    } else if (s.dtype == 1) {                                      \
      switch (G_) {                                                     \
        case 1: FN<1, 1>(__VA_ARGS__); break;                       \
        case 2: FN<1, 2>(__VA_ARGS__); break;                       \
        case 4: FN<1, 4>(__VA_ARGS__); break;                       \
        default: FN<1, 8>(__VA_ARGS__); break;                      \
      }                                                                 \
    } else {                                                            \
      switch (G_) {                                                     \
        case 1: FN<2, 1>(__VA_ARGS__); break;                        \
        case 2: FN<2, 2>(__VA_ARGS__); break;                        \
        case 4: FN<2, 4>(__VA_ARGS__); break;                        \
        default: FN<2, 8>(__VA_ARGS__); break;                       \
      }                                                                 \
    }                                                                   \
  } while (0)

constexpr int kScorerQuest = 0, kScorerMean = 1;

// A predicted set's per-row budget as the kernels take it (policy 0: fixed).
struct BudgetDev {
  int policy = 0, top_k = 0, k_min = 1;
  float beta = 0.f, c = 0.f;
  const int32_t* missed_prev = nullptr;
};
inline BudgetDev budget_dev(const prr_budget* b) {
  BudgetDev d;
  if (b && b->policy != PRR_BUDGET_FIXED) {
    d.policy = b->policy;
    d.top_k = b->top_k;
    d.k_min = b->k_min;
    d.beta = b->beta;
    d.c = b->c;
    d.missed_prev = b->missed_prev;
  }
  return d;
}
// Standalone budgeted prediction (with update: the EMA update first; then the per-row size, the top-k_r and the -1
// padding): one workgroup per row, rows of at most 32768 blocks.
prr_status launch_predict_budget(const prr_shape& s, const float* scores, float* ema, float alpha, int first, int cap,
                                 const BudgetDev& bp, int32_t* pred_next, bool update, hipStream_t stream);

// Tokens of the last block (block_size unless the sequence ends inside it).
inline int last_block_len(const prr_shape& s) {
  return s.ctx_len > 0 ? s.ctx_len - (s.n_blocks - 1) * s.block_size : s.block_size;
}
// Tokens of block n of a sequence whose last block N - 1 holds last_len tokens.
__host__ __device__ inline int block_len(int n, int N, int bs, int last_len) { return n == N - 1 ? last_len : bs; }

prr_status launch_append(const prr_shape& s, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* table, void* summ, hipStream_t stream);
prr_status launch_summaries(const prr_shape& s, const void* k_cache, const int32_t* table, const int32_t* ids,
                            int64_t n_jobs, void* summ, hipStream_t stream);
// Scores; with ema != nullptr also the EMA update (first != 0: ema = scores).
prr_status launch_score(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema, float alpha,
                        int first, hipStream_t stream);
// Top-K of each row (with ema != nullptr: of the EMA after its update). With cand != nullptr (a candidate region of
// topk_cand_bytes) rows longer than kTopkSplitMinN are split into segments, then merged.
prr_status launch_topk(const prr_shape& s, const float* values, float* ema, float alpha, int first, int k,
                       int32_t* out_idx, hipStream_t stream, void* cand = nullptr);
constexpr int kTopkSplitMinN = 8192;   // shorter rows take one workgroup each
constexpr int kTopkSeg1024 = 4096;     // segment of a 1024-thread workgroup (4 values per thread)
struct TopkCand {
  uint32_t* key;
  int32_t* idx;
  int64_t cap;   // candidate slots per row
};
size_t topk_cand_row_capacity(int N);
size_t topk_cand_bytes(const prr_shape& s);   // one candidate region (0 when rows are never split)
bool topk_split_on(int N, int K, int seg);
TopkCand topk_cand_at(const prr_shape& s, void* region);
// The true top-K of the scores and the next predicted set (top-K' of the EMA, or a budgeted set) in one launch of
// top-K workgroups only (rows of at most 32768 values). ema_update: the launch updates the EMA from the scores first
// (alpha, first as for the scoring pass); otherwise the EMA is taken as already updated.
prr_status launch_topk_pair(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema, int kp,
                            int32_t* pred_next, const BudgetDev& bp, hipStream_t stream, bool ema_update = false,
                            float alpha = 0.f, int first = 0);
prr_status launch_speculate(const prr_shape& s, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                            hipStream_t stream);
prr_status launch_repair(const prr_shape& s, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* table, const int32_t* sel, int top_k, const int32_t* pred, int k_spec,
                         const float* partials, float* out, int32_t* n_missed, void* workspace, hipStream_t stream);
size_t repair_workspace_bytes(const prr_shape& s, int top_k);
// The resolved-page pipelined attention path: 16-token chunks never straddle a page, and a wave's group of at most
// 8 entries (or 4 speculation slots) spans at most 64 chunks.
bool p16_path(const prr_shape& s);
// Predicted slots per speculation wave: about four 16-token chunks per wave, while keeping >= 4096 waves in flight.
int spec_slots_per_wave(const prr_shape& s, int k_spec);
// The true set, the next predicted set and the speculation over pred in the fewest launches the shape allows. With
// ema_upd (a predicted set of fixed size) the workgroups that predict, or rank the EMA's segments, update the EMA
// from the scores first (alpha, first as for the scoring pass), so the scoring pass may write the scores alone.
prr_status launch_select_spec(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema,
                              int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                              const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                              hipStream_t stream, void* cand_t = nullptr, void* cand_p = nullptr,
                              void* cand_u = nullptr, const BudgetDev& bp = BudgetDev{}, bool ema_upd = false,
                              float alpha = 0.f, int first = 0);
// The two-launch step: scores (+ EMA) with speculation, then selection with the row-wise repair and merge.
bool two_launch_supported(const prr_shape& s, int top_k, int k_spec, int k_spec_next);
prr_status launch_score_spec(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema,
                             float alpha, int first, const void* kc, const void* vc, const int32_t* table,
                             const int32_t* pred, int k_spec, float* partials, hipStream_t stream);
// Selection launch that also attends the missed blocks (T \ P_t) per row, and optionally speculates over P_t, then
// the merge launch (missed-block record + speculated records of the hits -> out).
prr_status launch_select_missed(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema,
                                int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                                const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                                bool speculate, float* out, int32_t* n_missed, void* workspace, hipStream_t stream,
                                const BudgetDev& bp = BudgetDev{}, bool ema_upd = false, float alpha = 0.f,
                                int first = 0);
size_t select_missed_ws_bytes(const prr_shape& s, int top_k);
prr_status launch_flush(void* buf, size_t bytes, hipStream_t stream);
prr_status launch_stream_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);

}  // namespace prr
