// Query-aware block scoring and exact top-K selection (PRR abstract: attend only to the top-K KV blocks of each
// query; PRR reference list, Quest: block scores from per-block key min/max), and the EMA predictor's update and
// top-K' (PRR abstract: a light predictor built on an exponential moving average).
//
// score_kernel: Quest's group-summed block score (or the mean-key score) as a streaming GEMV over all CUs
//   (score_dev.h); optionally updates the EMA in the same pass.
// topk_kernel: one workgroup per (b, g) row, 512 threads up to 4096 values and 1024 beyond (topk_dev.h);
//   optionally updates the EMA first.
// topk_seg_kernel + topk_merge_kernel: the same top-K for long rows when a candidate workspace is given: one
//   workgroup per segment of 4096 values, then one per row over the segments' candidates.
// predict_budget_kernel: the next predicted set of each row under a per-row budget (topk_dev.h predict_row).
#include "score_dev.h"
#include "topk_dev.h"

namespace prr {

template <int DT, int G, bool EMA>
__global__ __launch_bounds__(256) void score_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ summ,
                                                    float* __restrict__ scores, int Hq, int Hkv, int N, int chunk,
                                                    float* __restrict__ ema, float alpha, int first, int scorer) {
  score_any<DT, G, EMA>(scorer, blockIdx.x, blockIdx.y, q, summ, scores, Hq, Hkv, N, chunk, ema, alpha, first);
}

template <int NT, int KPT, bool EMA>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ vals, float* __restrict__ ema,
                                                  float alpha, int first, int N, int K, int32_t* __restrict__ out,
                                                  int sink, int local) {
  const int64_t row = blockIdx.x;
  topk_row<NT, KPT, EMA>(vals + row * N, EMA ? ema + row * N : nullptr, alpha, first, N, K, out + row * K, nullptr,
                         Force{0, N, sink, local});
}

template <int KPT, bool EMA>
__global__ __launch_bounds__(1024) void topk_seg_kernel(const float* __restrict__ vals, float* __restrict__ ema,
                                                        float alpha, int first, int N, int K, int seg, int64_t cap,
                                                        uint32_t* __restrict__ ckey, int32_t* __restrict__ cidx,
                                                        int sink, int local) {
  const int64_t row = blockIdx.y;
  topk_segment<1024, KPT, EMA>(vals + row * N, EMA ? ema + row * N : nullptr, alpha, first, N, K, seg, blockIdx.x,
                               ckey + row * cap, cidx + row * cap, sink, local);
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(const uint32_t* __restrict__ ckey,
                                                        const int32_t* __restrict__ cidx, int64_t cap, int C, int K,
                                                        int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  topk_merge_row<NT, KPT>(ckey + row * cap, cidx + row * cap, C, K, out + row * K);
}

template <int NT, int KPT, bool EMA>
__global__ __launch_bounds__(NT) void predict_budget_kernel(const float* __restrict__ scores, float* __restrict__ ema,
                                                            float alpha, int first, int N, int cap, BudgetDev bp,
                                                            int32_t* __restrict__ out, int sink, int local) {
  const int64_t row = blockIdx.x;
  predict_row<NT, KPT, EMA>(scores + row * N, ema + row * N, alpha, first, N, cap, bp, row, out + row * cap,
                            Force{0, N, sink, local});
}

// The true set and the next predicted set in one launch, with nothing to speculate: workgroup r < rows selects the
// true top-K of row r, workgroup rows + r the top-K' of row r's EMA or its budgeted set. With EUP the EMA is updated
// here (e = s on the first step, else alpha e + (1 - alpha) s, the scoring pass's arithmetic) by the workgroup that
// selects from it, which reads the scores anyway; without, the scoring pass has updated it. The workgroups are sized
// for the top-K alone (no attention tile beside it), so all of them are resident at once.
template <int NT, int KPT, bool EUP>
__global__ __launch_bounds__(NT) void topk_pair_kernel(const float* __restrict__ scores, int K,
                                                       int32_t* __restrict__ sel, float* __restrict__ ema,
                                                       float alpha, int first, int Kp, int32_t* __restrict__ pred_next,
                                                       int rows, int N, int sink, int local, BudgetDev bp) {
  const int64_t r = blockIdx.x;
  if (r < rows) {
    topk_row<NT, KPT, false>(scores + r * N, nullptr, 0.f, 0, N, K, sel + r * K, nullptr, Force{0, N, sink, local});
    return;
  }
  const int64_t rr = r - rows;
  if (bp.policy != 0)
    predict_row<NT, KPT, EUP>(scores + rr * N, ema + rr * N, alpha, first, N, Kp, bp, rr, pred_next + rr * Kp,
                              Force{0, N, sink, local});
  else if (EUP)
    topk_row<NT, KPT, true>(scores + rr * N, ema + rr * N, alpha, first, N, Kp, pred_next + rr * Kp, nullptr,
                            Force{0, N, sink, local});
  else
    topk_row<NT, KPT, false>(ema + rr * N, nullptr, 0.f, 0, N, Kp, pred_next + rr * Kp, nullptr,
                             Force{0, N, sink, local});
}

// ---- launchers -----------------------------------------------------------------------------------------------------

template <int DT, int G>
static void score_launch(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema, float alpha,
                         int first, hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const int chunk = score_chunk_size(s, ema != nullptr);
  const dim3 grid((unsigned)((s.n_blocks + chunk - 1) / chunk), (unsigned)rows), blk(256);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* sm = static_cast<const uint8_t*>(summ);
  if (ema)
    score_kernel<DT, G, true><<<grid, blk, 0, st>>>(qq, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk,
                                                    ema, alpha, first, s.scorer);
  else
    score_kernel<DT, G, false><<<grid, blk, 0, st>>>(qq, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk,
                                                     nullptr, 0.f, 0, s.scorer);
}

prr_status launch_score(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema, float alpha,
                        int first, hipStream_t stream) {
  trace_begin(PRR_KERNEL_SCORE, stream);
  PRR_DISPATCH_DT_G(score_launch, s, q, summ, scores, ema, alpha, first, stream);
  trace_end(PRR_KERNEL_SCORE, stream);
  return check_launch("score");
}

// Rows of up to 4096 values take a 512-thread workgroup (fewer waves at each of the select's barriers), longer
// rows 1024 threads.
template <bool EMA>
static void topk_dispatch(int N, dim3 grid, const float* vals, float* ema, float alpha, int first, int K, int sink,
                          int local, int32_t* out, hipStream_t st) {
#define PRR_TOPK(NT, KPT) \
  topk_kernel<NT, KPT, EMA><<<grid, NT, 0, st>>>(vals, ema, alpha, first, N, K, out, sink, local)
  if (N <= 4096) {
    switch (topk_kpt_nt(N, 512)) {
      case 1: PRR_TOPK(512, 1); break;
      case 2: PRR_TOPK(512, 2); break;
      case 4: PRR_TOPK(512, 4); break;
      default: PRR_TOPK(512, 8); break;
    }
    return;
  }
  switch (topk_kpt(N)) {
    case 1: case 2: case 4: case 8: PRR_TOPK(1024, 8); break;
    case 16: PRR_TOPK(1024, 16); break;
    default: PRR_TOPK(1024, 32); break;
  }
#undef PRR_TOPK
}

size_t topk_cand_row_capacity(int N) {
  return N > kTopkSplitMinN ? (size_t)((N / 2 + 2048 + 3) & ~3) : 0;
}

size_t topk_cand_bytes(const prr_shape& s) {
  return (size_t)s.batch * s.n_kv_heads * topk_cand_row_capacity(s.n_blocks) * (sizeof(uint32_t) + sizeof(int32_t));
}

bool topk_split_on(int N, int K, int seg) {
  // the merge holds at most 16 candidates per thread of a 1024-thread workgroup
  return N > kTopkSplitMinN && K <= seg / 2 && topk_split(N, K, seg).C <= 16 * 1024;
}

TopkCand topk_cand_at(const prr_shape& s, void* region) {
  const int64_t cap = (int64_t)topk_cand_row_capacity(s.n_blocks);
  auto* k = static_cast<uint32_t*>(region);
  return TopkCand{k, reinterpret_cast<int32_t*>(k + (int64_t)s.batch * s.n_kv_heads * cap), cap};
}

template <bool EMA>
static void topk_split_launch(const prr_shape& s, const float* vals, float* ema, float alpha, int first, int K,
                              int32_t* out, const TopkCand& c, hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const TopkSplit p = topk_split(s.n_blocks, K, kTopkSeg1024);
  topk_seg_kernel<4, EMA><<<dim3((unsigned)p.S, (unsigned)rows), 1024, 0, st>>>(vals, ema, alpha, first, s.n_blocks,
                                                                                K, p.seg, c.cap, c.key, c.idx,
                                                                                s.sink_blocks, s.local_blocks);
  const dim3 grid((unsigned)rows);
#define PRR_MERGE(NT, KPT) topk_merge_kernel<NT, KPT><<<grid, NT, 0, st>>>(c.key, c.idx, c.cap, p.C, K, out)
  if (p.C <= 4096) {   // 512 threads, as for short rows
    switch (topk_kpt_nt(p.C, 512)) {
      case 1: case 2: case 4: PRR_MERGE(512, 4); break;
      default: PRR_MERGE(512, 8); break;
    }
  } else {
    switch (topk_kpt(p.C)) {
      case 1: case 2: case 4: case 8: PRR_MERGE(1024, 8); break;
      default: PRR_MERGE(1024, 16); break;   // C <= 16384
    }
  }
#undef PRR_MERGE
}

template <bool EMA>
static void predict_budget_dispatch(const prr_shape& s, const float* scores, float* ema, float alpha, int first,
                                    int cap, const BudgetDev& bp, int32_t* pred_next, hipStream_t st) {
  const int N = s.n_blocks;
  const dim3 grid((unsigned)(s.batch * s.n_kv_heads));
#define PRR_PREDICT(NT, KPT)                                                                                       \
  predict_budget_kernel<NT, KPT, EMA><<<grid, NT, 0, st>>>(scores, ema, alpha, first, N, cap, bp, pred_next,       \
                                                           s.sink_blocks, s.local_blocks)
  if (N <= 4096) {
    switch (topk_kpt_nt(N, 512)) {
      case 1: PRR_PREDICT(512, 1); break;
      case 2: PRR_PREDICT(512, 2); break;
      case 4: PRR_PREDICT(512, 4); break;
      default: PRR_PREDICT(512, 8); break;
    }
  } else {
    switch (topk_kpt(N)) {
      case 1: case 2: case 4: case 8: PRR_PREDICT(1024, 8); break;
      case 16: PRR_PREDICT(1024, 16); break;
      default: PRR_PREDICT(1024, 32); break;   // N <= 32768
    }
  }
#undef PRR_PREDICT
}

prr_status launch_predict_budget(const prr_shape& s, const float* scores, float* ema, float alpha, int first, int cap,
                                 const BudgetDev& bp, int32_t* pred_next, bool update, hipStream_t st) {
  trace_begin(PRR_KERNEL_EMA_TOPK, st);
  if (update)
    predict_budget_dispatch<true>(s, scores, ema, alpha, first, cap, bp, pred_next, st);
  else
    predict_budget_dispatch<false>(s, scores, ema, alpha, first, cap, bp, pred_next, st);
  trace_end(PRR_KERNEL_EMA_TOPK, st);
  return check_launch("ema_predict (budget)");
}

prr_status launch_topk_pair(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema, int kp,
                            int32_t* pred_next, const BudgetDev& bp, hipStream_t st, bool ema_update, float alpha,
                            int first) {
  const int N = s.n_blocks, rows = s.batch * s.n_kv_heads;
  const dim3 grid((unsigned)(2 * rows));
  float* e = const_cast<float*>(ema);   // written only with ema_update
#define PRR_PAIR(NT, KPT)                                                                                          \
  (ema_update ? topk_pair_kernel<NT, KPT, true> : topk_pair_kernel<NT, KPT, false>)<<<grid, NT, 0, st>>>(         \
      scores, k, sel, e, alpha, first, kp, pred_next, rows, N, s.sink_blocks, s.local_blocks, bp)
  trace_begin(PRR_KERNEL_SELECT_TOPK, st);
  if (N <= 4096) {
    switch (topk_kpt_nt(N, 512)) {
      case 1: case 2: PRR_PAIR(512, 2); break;
      case 4: PRR_PAIR(512, 4); break;
      default: PRR_PAIR(512, 8); break;
    }
  } else {
    switch (topk_kpt(N)) {
      case 1: case 2: case 4: case 8: PRR_PAIR(1024, 8); break;
      case 16: PRR_PAIR(1024, 16); break;
      default: PRR_PAIR(1024, 32); break;   // N <= 32768
    }
  }
#undef PRR_PAIR
  trace_end(PRR_KERNEL_SELECT_TOPK, st);
  return check_launch("select (true and predicted sets)");
}

prr_status launch_topk(const prr_shape& s, const float* values, float* ema, float alpha, int first, int k,
                       int32_t* out_idx, hipStream_t stream, void* cand) {
  const int kid = ema ? PRR_KERNEL_EMA_TOPK : PRR_KERNEL_SELECT_TOPK;
  trace_begin(kid, stream);
  if (cand && topk_split_on(s.n_blocks, k, kTopkSeg1024)) {
    const TopkCand c = topk_cand_at(s, cand);
    if (ema)
      topk_split_launch<true>(s, values, ema, alpha, first, k, out_idx, c, stream);
    else
      topk_split_launch<false>(s, values, nullptr, alpha, first, k, out_idx, c, stream);
  } else {
    const dim3 grid((unsigned)(s.batch * s.n_kv_heads));
    if (ema)
      topk_dispatch<true>(s.n_blocks, grid, values, ema, alpha, first, k, s.sink_blocks, s.local_blocks, out_idx,
                          stream);
    else
      topk_dispatch<false>(s.n_blocks, grid, values, nullptr, alpha, first, k, s.sink_blocks, s.local_blocks,
                           out_idx, stream);
  }
  trace_end(kid, stream);
  return check_launch(ema ? "ema_predict" : "select_topk");
}

}  // namespace prr
