// Scoring and speculation in one launch (PRR abstract: speculate over the predicted blocks while selection is in
// flight). Workgroups [0, n_spec_wg) run speculation (one wave per predicted slot); the rest score the block
// summaries. Both roles stream HBM concurrently on the same launch, so the overlap needs no second queue and no
// cross-stream synchronisation.
#include "attn_wave.h"
#include "score_dev.h"

namespace prr {

template <int DT, int G>
__global__ __launch_bounds__(256) void score_spec_kernel(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ summ, float* __restrict__ scores,
                                                         int chunk, int score_gx, const uint8_t* __restrict__ kc,
                                                         const uint8_t* __restrict__ vc,
                                                         const int32_t* __restrict__ table,
                                                         const int32_t* __restrict__ pred, int k_spec,
                                                         float* __restrict__ partials, int n_spec_wg,
                                                         int64_t spec_total, int Hq, int Hkv, int N, int bs, int page,
                                                         int pps, float qscale) {
  if ((int)blockIdx.x < n_spec_wg) {
    const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s < spec_total)
      speculate_slot<DT, G>(s, threadIdx.x & 63, q, kc, vc, table, pred, k_spec, partials, Hq, Hkv, N, bs, page,
                            pps, qscale);
    return;
  }
  const int sb = (int)blockIdx.x - n_spec_wg;
  score_chunk<DT, G>(sb % score_gx, sb / score_gx, q, summ, scores, Hq, Hkv, N, chunk);
}

template <int DT, int G>
static void score_spec_launch(const prr_shape& s, const void* q, const void* summ, float* scores, const void* kc,
                              const void* vc, const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                              hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const int chunk = score_chunk_size(s);
  const int gx = (s.n_blocks + chunk - 1) / chunk;
  const int64_t spec_total = (int64_t)rows * k_spec;
  const int n_spec_wg = (int)((spec_total + 3) / 4);
  const unsigned grid = (unsigned)(n_spec_wg + (int64_t)gx * rows);
  score_spec_kernel<DT, G><<<dim3(grid), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(summ), scores, chunk, gx,
      static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, pred, k_spec, partials, n_spec_wg,
      spec_total, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size, s.pages_per_seq,
      s.softmax_scale * kLog2e);
}

prr_status launch_score_spec(const prr_shape& s, const void* q, const void* summ, float* scores, const void* kc,
                             const void* vc, const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                             hipStream_t stream) {
  trace_begin(PRR_KERNEL_SCORE, stream);
  PRR_DISPATCH_DT_G(score_spec_launch, s, q, summ, scores, kc, vc, table, pred, k_spec, partials, stream);
  trace_end(PRR_KERNEL_SCORE, stream);
  return check_launch("score_speculate");
}

}  // namespace prr
