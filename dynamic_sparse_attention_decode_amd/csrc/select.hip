// Query-aware block scoring and exact top-K selection (PRR abstract: attend only to the top-K KV blocks of each
// query; PRR reference list, Quest: block scores from per-block key min/max), and the EMA predictor's update and
// top-K' (PRR abstract: "lightweight EMA-based predictor").
//
// score_kernel: Quest's group-summed block score as a streaming GEMV over all CUs (score_dev.h); optionally updates
//   the EMA in the same pass.
// topk_kernel: one 1024-thread workgroup per (b, g) row (topk_dev.h); optionally updates the EMA first.
#include "score_dev.h"
#include "topk_dev.h"

namespace prr {

template <int DT, int G, bool EMA>
__global__ __launch_bounds__(256) void score_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ summ,
                                                    float* __restrict__ scores, int Hq, int Hkv, int N, int chunk,
                                                    float* __restrict__ ema, float alpha, int first) {
  score_chunk<DT, G, EMA>(blockIdx.x, blockIdx.y, q, summ, scores, Hq, Hkv, N, chunk, ema, alpha, first);
}

template <int NT, int KPT, bool EMA>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ vals, float* __restrict__ ema,
                                                  float alpha, int first, int N, int K, int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  topk_row<NT, KPT, EMA>(vals + row * N, EMA ? ema + row * N : nullptr, alpha, first, N, K, out + row * K);
}

// ---- launchers -----------------------------------------------------------------------------------------------------

template <int DT, int G>
static void score_launch(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema, float alpha,
                         int first, hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const int chunk = score_chunk_size(s);
  const dim3 grid((unsigned)((s.n_blocks + chunk - 1) / chunk), (unsigned)rows), blk(256);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* sm = static_cast<const uint8_t*>(summ);
  if (ema)
    score_kernel<DT, G, true><<<grid, blk, 0, st>>>(qq, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk,
                                                    ema, alpha, first);
  else
    score_kernel<DT, G, false><<<grid, blk, 0, st>>>(qq, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk,
                                                     nullptr, 0.f, 0);
}

prr_status launch_score(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema, float alpha,
                        int first, hipStream_t stream) {
  trace_begin(PRR_KERNEL_SCORE, stream);
  PRR_DISPATCH_DT_G(score_launch, s, q, summ, scores, ema, alpha, first, stream);
  trace_end(PRR_KERNEL_SCORE, stream);
  return check_launch("score");
}

template <bool EMA>
static void topk_dispatch(int kpt, dim3 grid, const float* vals, float* ema, float alpha, int first, int N, int K,
                          int32_t* out, hipStream_t st) {
  switch (kpt) {
    case 1: topk_kernel<1024, 1, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 2: topk_kernel<1024, 2, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 4: topk_kernel<1024, 4, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 8: topk_kernel<1024, 8, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 16: topk_kernel<1024, 16, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    default: topk_kernel<1024, 32, EMA><<<grid, 1024, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
  }
}

prr_status launch_topk(const prr_shape& s, const float* values, float* ema, float alpha, int first, int k,
                       int32_t* out_idx, hipStream_t stream) {
  const int kpt = topk_kpt(s.n_blocks);
  const dim3 grid((unsigned)(s.batch * s.n_kv_heads));
  const int kid = ema ? PRR_KERNEL_EMA_TOPK : PRR_KERNEL_SELECT_TOPK;
  trace_begin(kid, stream);
  if (ema)
    topk_dispatch<true>(kpt, grid, values, ema, alpha, first, s.n_blocks, k, out_idx, stream);
  else
    topk_dispatch<false>(kpt, grid, values, nullptr, alpha, first, s.n_blocks, k, out_idx, stream);
  trace_end(kid, stream);
  return check_launch(ema ? "ema_predict" : "select_topk");
}

}  // namespace prr
