// Speculation co-scheduled with selection inside one launch (PRR abstract: speculate over the predicted blocks while
// selection is in flight), so the overlap needs no second queue and no cross-stream synchronisation.
//
// select_spec_kernel (512 threads per workgroup): workgroups [0, rows) select the true top-K of the scores,
// [rows, 2 rows) the next step's predicted set (top-K' of the EMA, which the scoring launch has already updated), and
// the rest run speculation over the current predicted set, one wave per slot. Selection keeps one workgroup per row
// busy and is bound by latency, so the speculative loads use bandwidth that would otherwise sit idle.
#include "attn_wave.h"
#include "topk_dev.h"

namespace prr {

constexpr int kSelSpecThreads = 512;   // 8 waves: room for the speculation tile's registers

template <int KPT, int DT, int G>
__global__ __launch_bounds__(kSelSpecThreads) void select_spec_kernel(const float* __restrict__ scores, int K,
                                                           int32_t* __restrict__ sel, const float* __restrict__ ema,
                                                           int Kp_next, int32_t* __restrict__ pred_next, int n_sel_wg,
                                                           const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ kc,
                                                           const uint8_t* __restrict__ vc,
                                                           const int32_t* __restrict__ table,
                                                           const int32_t* __restrict__ pred, int k_spec,
                                                           float* __restrict__ partials, int64_t spec_total, int Hq,
                                                           int Hkv, int N, int bs, int page, int pps, float qscale,
                                                           int rows) {
  const int64_t r = blockIdx.x;
  if (r < n_sel_wg) {
    if (r < rows)
      topk_row<kSelSpecThreads, KPT, false>(scores + r * N, nullptr, 0.f, 0, N, K, sel + r * K);
    else
      topk_row<kSelSpecThreads, KPT, false>(ema + (r - rows) * N, nullptr, 0.f, 0, N, Kp_next,
                                            pred_next + (r - rows) * Kp_next);
    return;
  }
  const int64_t s = (r - n_sel_wg) * (kSelSpecThreads / 64) + (threadIdx.x >> 6);
  if (s < spec_total)
    speculate_slot<DT, G>(s, threadIdx.x & 63, q, kc, vc, table, pred, k_spec, partials, Hq, Hkv, N, bs, page, pps,
                          qscale);
}

template <int DT, int G>
static void select_spec_launch(const prr_shape& s, const float* scores, int K, int32_t* sel, const float* ema,
                               int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                               const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                               hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const int n_sel_wg = kp_next > 0 ? 2 * rows : rows;
  const int64_t spec_total = (int64_t)rows * k_spec;
  constexpr int WPG = kSelSpecThreads / 64;
  const int n_spec_wg = (int)((spec_total + WPG - 1) / WPG);
  const dim3 grid((unsigned)(n_sel_wg + n_spec_wg)), blk(kSelSpecThreads);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* kk = static_cast<const uint8_t*>(kc);
  const auto* vv = static_cast<const uint8_t*>(vc);
  const float qs = s.softmax_scale * kLog2e;
#define PRR_SELSPEC(KPT)                                                                                           \
  select_spec_kernel<KPT, DT, G><<<grid, blk, 0, st>>>(scores, K, sel, ema, kp_next, pred_next, n_sel_wg, qq, kk, vv, \
                                                       table, pred, k_spec, partials, spec_total, s.n_q_heads,       \
                                                       s.n_kv_heads, s.n_blocks, s.block_size, s.page_size,          \
                                                       s.pages_per_seq, qs, rows)
  // values per thread: a few register sizes cover every row length (larger than needed is correct, just slower)
  if (s.n_blocks <= 4 * kSelSpecThreads)
    PRR_SELSPEC(4);
  else if (s.n_blocks <= 16 * kSelSpecThreads)
    PRR_SELSPEC(16);
  else
    PRR_SELSPEC(64);
#undef PRR_SELSPEC
}

prr_status launch_select_spec(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema,
                              int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                              const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                              hipStream_t stream) {
  trace_begin(PRR_KERNEL_SELECT_TOPK, stream);
  PRR_DISPATCH_DT_G(select_spec_launch, s, scores, k, sel, ema, kp_next, pred_next, q, kc, vc, table, pred, k_spec,
                    partials, stream);
  trace_end(PRR_KERNEL_SELECT_TOPK, stream);
  return check_launch("select_speculate");
}

}  // namespace prr
