// Speculation co-scheduled with selection inside one launch (PRR abstract: speculate over the predicted blocks while
// selection is in flight), so the overlap needs no second queue and no cross-stream synchronisation.
//
// select_spec_kernel (512 threads per workgroup): workgroups [0, rows) select the true top-K of the scores,
// [rows, 2 rows) the next step's predicted set (top-K' of the EMA, which the scoring launch has already updated), and
// the rest run speculation over the current predicted set, one wave per slot. Selection keeps one workgroup per row
// busy and is bound by latency, so the speculative loads use bandwidth that would otherwise sit idle.
//
// Long rows (given candidate regions): seg_spec_kernel's first workgroups select the top-K of each segment of 2048
// scores and the top-K' of each segment of the EMA (in the decode step with a fixed budget they update that segment
// of the EMA from the scores first), the rest speculate as the standalone speculation kernel does (256-thread
// workgroups, several slots per wave); merge2_kernel then selects each row's T and P_{t+1} from the segments'
// candidates (topk_dev.h).
#include <atomic>

#include "attn_wave.h"
#include "topk_dev.h"

namespace prr {

constexpr int kSelSpecThreads = 512;   // 8 waves: room for the speculation tile's registers

// Compute units of the current device (queried once per device; 256 on MI355X).
static int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int NT, int KPT, int DT, int G>
__global__ __launch_bounds__(NT) void select_spec_kernel(const float* __restrict__ scores, int K,
                                                           int32_t* __restrict__ sel, const float* __restrict__ ema,
                                                           int Kp_next, int32_t* __restrict__ pred_next, int n_sel_wg,
                                                           const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ kc,
                                                           const uint8_t* __restrict__ vc,
                                                           const int32_t* __restrict__ table,
                                                           const int32_t* __restrict__ pred, int k_spec,
                                                           float* __restrict__ partials, int64_t spec_total, int Hq,
                                                           int Hkv, int N, int bs, int page, int pps, float qscale,
                                                           int rows, int last_len, int sink, int local,
                                                           BudgetDev bp, int ema_upd, float alpha, int first) {
  const int64_t r = blockIdx.x;
  if (r < n_sel_wg) {
    const Force force{0, N, sink, local};
    if (r < rows) {
      topk_row<NT, KPT, false>(scores + r * N, nullptr, 0.f, 0, N, K, sel + r * K, nullptr, force);
      return;
    }
    const int64_t rr = r - rows;   // the next predicted set of row rr
    float* erow = const_cast<float*>(ema) + rr * N;
    int32_t* prow = pred_next + rr * Kp_next;
    if (ema_upd) {   // fixed budget: update the row's EMA from the scores, then take its top-K'
      topk_row<NT, KPT, true>(scores + rr * N, erow, alpha, first, N, Kp_next, prow, nullptr, force);
    } else {
      if constexpr (KPT <= 16) {   // budgeted rows are routed elsewhere beyond 8192 blocks
        if (bp.policy != 0) {
          predict_row<NT, KPT, false>(scores + rr * N, erow, 0.f, 0, N, Kp_next, bp, rr, prow, force);
          return;
        }
      }
      topk_row<NT, KPT, false>(erow, nullptr, 0.f, 0, N, Kp_next, prow, nullptr, force);
    }
    return;
  }
  const int64_t s = (r - n_sel_wg) * (NT / 64) + (threadIdx.x >> 6);
  if (s < spec_total)
    speculate_slot<DT, G>(s, threadIdx.x & 63, q, kc, vc, table, pred, k_spec, partials, Hq, Hkv, N, bs, page, pps,
                          qscale, last_len);
}

constexpr int kSegSpecThreads = 256;                // the standalone speculation kernel's workgroup
constexpr int kSelSpecSeg = 8 * kSegSpecThreads;    // segment of one workgroup: 2048 values, 8 per thread

template <int DT, int G, bool P16>
__global__ __launch_bounds__(kSegSpecThreads, 3) void seg_spec_kernel(const float* __restrict__ scores, int K,
                                                           const float* __restrict__ ema, int Kp_next, int S,
                                                           int n_seg_wg, TopkCand ct, TopkCand cp,
                                                           const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ kc,
                                                           const uint8_t* __restrict__ vc,
                                                           const int32_t* __restrict__ table,
                                                           const int32_t* __restrict__ pred, int k_spec,
                                                           float* __restrict__ partials, int spw, int wpr,
                                                           int64_t spec_waves, int Hq, int Hkv, int N, int bs,
                                                           int page, int pps, float qscale, int rows, int last_len,
                                                           int sink, int local, int Ke, TopkCand cu, float conf_c,
                                                           int ema_upd, float alpha, int first) {
  const int64_t r = blockIdx.x;
  if (r < n_seg_wg) {
    const int64_t job = r / S;
    const int seg = (int)(r % S);
    if (job < rows) {
      topk_segment<kSegSpecThreads, 8, false>(scores + job * N, nullptr, 0.f, 0, N, K, kSelSpecSeg, seg,
                                              ct.key + job * ct.cap, ct.idx + job * ct.cap, sink, local);
    } else if (job < 2 * rows) {   // the EMA's top-Ke of the segment (Ke = K' or, for a confidence budget, K)
      const int64_t rr = job - rows;
      if (ema_upd)   // update the segment's EMA from the scores first, then rank the updated values
        topk_segment<kSegSpecThreads, 8, true>(scores + rr * N, const_cast<float*>(ema) + rr * N, alpha, first, N,
                                               Ke, kSelSpecSeg, seg, cp.key + rr * cp.cap, cp.idx + rr * cp.cap,
                                               sink, local);
      else
        topk_segment<kSegSpecThreads, 8, false>(ema + rr * N, nullptr, 0.f, 0, N, Ke, kSelSpecSeg, seg,
                                                cp.key + rr * cp.cap, cp.idx + rr * cp.cap, sink, local);
    } else {   // a confidence budget's optimistic scores: the segment's top-K'
      const int64_t rr = job - 2 * rows;
      topk_segment<kSegSpecThreads, 8, false>(ema + rr * N, nullptr, 0.f, 0, N, Kp_next, kSelSpecSeg, seg,
                                              cu.key + rr * cu.cap, cu.idx + rr * cu.cap, sink, local,
                                              scores + rr * N, conf_c);
    }
    return;
  }
  // speculation as the standalone kernel does it: spw consecutive slots per wave
  const int64_t w = (r - n_seg_wg) * (kSegSpecThreads / 64) + (threadIdx.x >> 6);
  if (w >= spec_waves) return;
  const int64_t rowid = w / wpr;
  const int j0 = (int)(w - rowid * wpr) * spw;
  speculate_slots<DT, G, P16>(rowid, j0, min(k_spec, j0 + spw), threadIdx.x & 63, q, kc, vc, table, pred, k_spec,
                              partials, Hq, Hkv, N, bs, page, pps, qscale, last_len);
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void merge2_kernel(TopkCand ct, int Ct, int K, int32_t* __restrict__ sel,
                                                    TopkCand cp, int Cp, int Kp_next, int32_t* __restrict__ pred_next,
                                                    int rows, BudgetDev bp, TopkCand cu, int Cu) {
  const int64_t r = blockIdx.x;
  if (r < rows) {
    topk_merge_row<NT, KPT>(ct.key + r * ct.cap, ct.idx + r * ct.cap, Ct, K, sel + r * K);
    return;
  }
  const int64_t rr = r - rows;
  if (bp.policy != 0)
    topk_merge_budget_row<NT, KPT>(cp.key + rr * cp.cap, cp.idx + rr * cp.cap, Cp, cu.key + rr * cu.cap,
                                   cu.idx + rr * cu.cap, Cu, Kp_next, bp, rr, pred_next + rr * Kp_next);
  else
    topk_merge_row<NT, KPT>(cp.key + rr * cp.cap, cp.idx + rr * cp.cap, Cp, Kp_next, pred_next + rr * Kp_next);
}

// ema_upd: the EMA-segment workgroups update the EMA from the scores (alpha, first) before they rank it.
template <int DT, int G>
static void seg_spec_launch(const prr_shape& s, const float* scores, int K, int32_t* sel, const float* ema,
                            int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                            const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                            const TopkCand& ct, const TopkCand& cp, const TopkCand& cu, const BudgetDev& bp,
                            hipStream_t st, bool ema_upd = false, float alpha = 0.f, int first = 0) {
  const int rows = s.batch * s.n_kv_heads;
  const bool conf = kp_next > 0 && bp.policy == 2;
  const int ke = conf ? bp.top_k : kp_next;   // EMA candidates per segment: K for the confidence rule's theta
  const TopkSplit pt = topk_split(s.n_blocks, K, kSelSpecSeg);
  const TopkSplit pp = topk_split(s.n_blocks, kp_next > 0 ? ke : 1, kSelSpecSeg);
  const TopkSplit pu = topk_split(s.n_blocks, kp_next > 0 ? kp_next : 1, kSelSpecSeg);
  const int n_seg_wg = (kp_next > 0 ? (conf ? 3 : 2) : 1) * rows * pt.S;
  const int spw = k_spec > 0 ? spec_slots_per_wave(s, k_spec) : 1;
  const int wpr = (k_spec + spw - 1) / spw;
  const int64_t spec_waves = (int64_t)rows * wpr;
  constexpr int WPG = kSegSpecThreads / 64;
  const int n_spec_wg = (int)((spec_waves + WPG - 1) / WPG);
  auto kern = p16_path(s) ? seg_spec_kernel<DT, G, true> : seg_spec_kernel<DT, G, false>;
  kern<<<dim3((unsigned)(n_seg_wg + n_spec_wg)), kSegSpecThreads, 0, st>>>(
      scores, K, ema, kp_next, pt.S, n_seg_wg, ct, cp, static_cast<const uint8_t*>(q),
      static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, pred, k_spec, partials, spw, wpr,
      spec_waves, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size, s.pages_per_seq,
      s.softmax_scale * kLog2e, rows, last_block_len(s), s.sink_blocks, s.local_blocks, ke, cu, bp.c,
      ema_upd ? 1 : 0, alpha, first);
  int cmax = pt.C;
  if (kp_next > 0) cmax = max(cmax, max(pp.C, conf ? pu.C : 0));
  const dim3 grid((unsigned)((kp_next > 0 ? 2 : 1) * rows));
#define PRR_MERGE2(NT, KPT)                                                                                        \
  merge2_kernel<NT, KPT><<<grid, NT, 0, st>>>(ct, pt.C, K, sel, cp, pp.C, kp_next, pred_next, rows,               \
                                              kp_next > 0 ? bp : BudgetDev{}, cu, pu.C)
  if (cmax <= 4096) {   // 512 threads, as for short rows
    switch (topk_kpt_nt(cmax, 512)) {
      case 1: case 2: case 4: PRR_MERGE2(512, 4); break;
      default: PRR_MERGE2(512, 8); break;
    }
  } else {
    switch (topk_kpt(cmax)) {
      case 1: case 2: case 4: case 8: PRR_MERGE2(1024, 8); break;
      default: PRR_MERGE2(1024, 16); break;   // C <= 16384 (topk_split_on)
    }
  }
#undef PRR_MERGE2
}

template <int DT, int G>
static void select_spec_launch(const prr_shape& s, const float* scores, int K, int32_t* sel, const float* ema,
                               int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                               const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                               const BudgetDev& bp, hipStream_t st, bool ema_upd, float alpha, int first) {
  const int rows = s.batch * s.n_kv_heads;
  const int n_sel_wg = kp_next > 0 ? 2 * rows : rows;
  const int64_t spec_total = (int64_t)rows * k_spec;
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* kk = static_cast<const uint8_t*>(kc);
  const auto* vv = static_cast<const uint8_t*>(vc);
  const float qs = s.softmax_scale * kLog2e;
#define PRR_SELSPEC(NT, KPT)                                                                                       \
  select_spec_kernel<NT, KPT, DT, G><<<dim3((unsigned)(n_sel_wg + (spec_total + NT / 64 - 1) / (NT / 64))), NT, 0,  \
                                       st>>>(scores, K, sel, ema, kp_next, pred_next, n_sel_wg, qq, kk, vv,           \
                                                       table, pred, k_spec, partials, spec_total, s.n_q_heads,       \
                                                       s.n_kv_heads, s.n_blocks, s.block_size, s.page_size,          \
                                                       s.pages_per_seq, qs, rows, last_block_len(s),            \
                                                       s.sink_blocks, s.local_blocks, bp, ema_upd ? 1 : 0, alpha,    \
                                                       first)
  // Rows of up to 2048 blocks whose launch of 512-thread workgroups (one per CU at these register counts) would not
  // be resident at once take 256-thread workgroups (three per CU), so that every speculation wave starts in the
  // first round (131K batch, same-box A/B over two runs: PRR step 49.5 -> 45.7 us); where the 512-thread launch fits,
  // it stays, since its top-K workgroups are faster (32K layer: 20.8 against 21.1 us with 256 threads).
  const int64_t wg512 = n_sel_wg + (spec_total + kSelSpecThreads / 64 - 1) / (kSelSpecThreads / 64);
  // values per thread: a few register sizes cover every row length (larger than needed is correct, just slower)
  if (s.n_blocks <= 2048 && wg512 > device_cus())
    PRR_SELSPEC(256, 8);
  else if (s.n_blocks <= 4 * kSelSpecThreads)
    PRR_SELSPEC(kSelSpecThreads, 4);
  else if (s.n_blocks <= 16 * kSelSpecThreads)
    PRR_SELSPEC(kSelSpecThreads, 16);
  else
    PRR_SELSPEC(kSelSpecThreads, 64);
#undef PRR_SELSPEC
}

prr_status launch_select_spec(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema,
                              int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                              const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                              hipStream_t stream, void* cand_t, void* cand_p, void* cand_u, const BudgetDev& bp,
                              bool ema_upd, float alpha, int first) {
  // nothing to speculate or predict: the selection alone, exactly as the serialized step runs it
  if (k_spec == 0 && kp_next == 0) return launch_topk(s, scores, nullptr, 0.f, 0, k, sel, stream, cand_t);
  if (ema_upd && (kp_next == 0 || !ema || bp.policy != 0)) {
    set_error("select_speculate: the EMA update in the selection launch needs a predicted set of fixed size");
    return PRR_EINVAL;
  }
  // long rows by segments (with the candidate regions): T, the EMA's candidates and, for a confidence budget, the
  // optimistic scores' candidates; the merge launch applies the budget
  const int ke = bp.policy == 2 ? bp.top_k : kp_next;
  const bool split = cand_t && cand_p && (bp.policy != 2 || cand_u) && topk_split_on(s.n_blocks, k, kSelSpecSeg) &&
                     (kp_next == 0 || (topk_split_on(s.n_blocks, kp_next, kSelSpecSeg) &&
                                       topk_split_on(s.n_blocks, ke, kSelSpecSeg)));
  // nothing to speculate: the true and predicted sets in one launch of top-K workgroups only
  if (k_spec == 0 && !split)
    return launch_topk_pair(s, scores, k, sel, ema, kp_next, pred_next, bp, stream, ema_upd, alpha, first);
  if (bp.policy != 0 && kp_next > 0 && !split && s.n_blocks > 16 * kSelSpecThreads) {
    // budgeted rows this long take their own launch of 1024-thread workgroups, which reads the EMA as it stands
    const prr_status st = launch_select_spec(s, scores, k, sel, nullptr, 0, nullptr, q, kc, vc, table, pred, k_spec,
                                             partials, stream, cand_t, cand_p, cand_u, BudgetDev{});
    if (st != PRR_OK) return st;
    return launch_predict_budget(s, scores, const_cast<float*>(ema), 0.f, 0, kp_next, bp, pred_next, false, stream);
  }
  trace_begin(PRR_KERNEL_SELECT_TOPK, stream);
  if (split) {
    const TopkCand ct = topk_cand_at(s, cand_t), cp = topk_cand_at(s, cand_p);
    const TopkCand cu = cand_u ? topk_cand_at(s, cand_u) : TopkCand{nullptr, nullptr, 0};
    PRR_DISPATCH_DT_G(seg_spec_launch, s, scores, k, sel, ema, kp_next, pred_next, q, kc, vc, table, pred, k_spec,
                      partials, ct, cp, cu, bp, stream, ema_upd, alpha, first);
  } else {
    PRR_DISPATCH_DT_G(select_spec_launch, s, scores, k, sel, ema, kp_next, pred_next, q, kc, vc, table, pred, k_spec,
                      partials, bp, stream, ema_upd, alpha, first);
  }
  trace_end(PRR_KERNEL_SELECT_TOPK, stream);
  return check_launch("select_speculate");
}

}  // namespace prr
