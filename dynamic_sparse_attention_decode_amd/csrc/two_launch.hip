// The PRR decode step in two launches (PRR abstract: speculate over the predicted blocks while selection is in
// flight, then repair the missed blocks once the true set is known).
//
// score_spec_kernel: workgroups [0, n_spec_wg) speculate over P_t (per-block partial records, one wave per few
//   slots); the rest compute the block scores (and update the EMA). Scoring reads the summaries and speculation reads
//   the predicted blocks, concurrently, so the speculative loads fill bandwidth that selection leaves unused.
// select_missed_kernel (512 threads): workgroup r < rows selects the true top-K of row r and then, in the same
//   workgroup, finds each entry of T in P_t; its 8 waves attend the missed blocks (T minus P_t) from the KV cache
//   and merge them in LDS into one partial record, and the slots of the hits go to the workspace; blocks of P_t
//   outside T never enter. Workgroups [rows, 2 rows) compute the next predicted set (top-K' of the updated EMA); the
//   rest, when asked, speculate over P_t.
// merge_hits_kernel: one workgroup per (row, head) merges the missed-block record with the speculated records of
//   the hits and writes out = O / l.
// With P_t empty the two launches are select-then-attend (the serialized path in two launches).
#include "attn_wave.h"
#include "score_dev.h"
#include "topk_dev.h"

namespace prr {

template <int DT, int G, bool EMA, bool P16>
__global__ __launch_bounds__(256, 3) void score_spec_kernel(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ summ, float* __restrict__ scores,
                                                         int chunk, int score_gx, float* __restrict__ ema, float alpha,
                                                         int first, const uint8_t* __restrict__ kc,
                                                         const uint8_t* __restrict__ vc,
                                                         const int32_t* __restrict__ table,
                                                         const int32_t* __restrict__ pred, int k_spec,
                                                         float* __restrict__ partials, int n_spec_wg, int spw, int wpr,
                                                         int64_t spec_waves, int Hq, int Hkv, int N, int bs, int page,
                                                         int pps, float qscale, int last_len, int scorer) {
  if ((int)blockIdx.x < n_spec_wg) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w < spec_waves) {
      const int64_t rowid = w / wpr;
      const int j0 = (int)(w - rowid * wpr) * spw;
      speculate_slots<DT, G, P16>(rowid, j0, min(k_spec, j0 + spw), threadIdx.x & 63, q, kc, vc, table, pred,
                                  k_spec, partials, Hq, Hkv, N, bs, page, pps, qscale, last_len);
    }
    return;
  }
  const int sb = (int)blockIdx.x - n_spec_wg;
  score_any<DT, G, EMA>(scorer, sb % score_gx, sb / score_gx, q, summ, scores, Hq, Hkv, N, chunk, ema, alpha, first);
}

constexpr int kSRThreads = 512;   // 8 waves: the attention tile keeps its full register budget
constexpr int kSRMaxK = 2048;     // largest top-K and predicted set handled in LDS

// Per-row workspace of the selection-and-repair launch: the slots of the hits (blocks of T found in P_t), their
// count, and the partial record of the missed blocks.
struct MissedWs {
  int32_t* hits;    // [rows][Kp]
  int32_t* cnt;     // [rows]
  float* mrec;      // [rows][RF]
  int Kp;
};

__host__ __device__ inline size_t missed_ws_layout(int64_t rows, int K, int RF, void* base, MissedWs* out) {
  const int Kp = (K + 3) & ~3;
  const size_t hits_b = (size_t)rows * Kp * 4;
  const size_t cnt_b = ((size_t)rows * 4 + 255) / 256 * 256;
  const size_t rec_b = (size_t)rows * RF * 4;
  if (out) {
    char* p = static_cast<char*>(base);
    out->hits = reinterpret_cast<int32_t*>(p);
    out->cnt = reinterpret_cast<int32_t*>(p + hits_b);
    out->mrec = reinterpret_cast<float*>(p + hits_b + cnt_b);
    out->Kp = Kp;
  }
  return hits_b + cnt_b + rec_b;
}

// Workgroup r < rows: true top-K of row r, then (same workgroup) the blocks of T missing from P_t are attended from
// the KV cache by the 8 waves and merged into one partial record of the row; the hits' slots go to the workspace for
// the merge launch. Workgroups [rows, rows + n_pwg): next predicted set (top-K' of the EMA, which with ema_upd they
// update from the scores first). The rest:
// speculation over P_t (one wave per slot) when spec_total > 0.
template <int KPT, int DT, int G>
__global__ __launch_bounds__(kSRThreads) void select_missed_kernel(
    const float* __restrict__ scores, int K, int32_t* __restrict__ sel, const float* __restrict__ ema, int Kp_next,
    int32_t* __restrict__ pred_next, const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const int32_t* __restrict__ table, const int32_t* __restrict__ pred, int k_spec,
    float* __restrict__ partials, int64_t spec_total, MissedWs ws, int32_t* __restrict__ n_missed, int Hq, int Hkv,
    int N, int bs, int page, int pps, float qscale, int rows, int n_pwg, int last_len, int sink, int local,
    BudgetDev bp, int ema_upd, float alpha, int first) {
  using W = Tile<DT, G>;
  constexpr int NW = kSRThreads / 64;
  constexpr int D = W::D;
  constexpr int RF = rec_floats(G, D);
  constexpr int ML = rec_ml(G);
  __shared__ int32_t s_T[kSRMaxK];
  __shared__ int32_t s_P[kSRMaxK];
  __shared__ int32_t s_list[kSRMaxK];   // slots of the hits, then ids of the missed blocks
  __shared__ uint32_t s_scan[NW];
  __shared__ int s_unsorted;
  __shared__ int s_kf;   // filled slots of P_t (a budgeted set ends in -1 slots)
  __shared__ float s_ml[NW][2 * G];
  __shared__ float s_o[NW][G * D];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (r >= rows + n_pwg) {   // speculation over P_t
    const int64_t s = (r - rows - n_pwg) * NW + wave;
    if (s < spec_total)
      speculate_slot<DT, G>(s, lane, q, kc, vc, table, pred, k_spec, partials, Hq, Hkv, N, bs, page, pps, qscale,
                            last_len);
    return;
  }
  if (r >= rows) {   // next step's predicted set
    const int64_t rr = r - rows;
    if (ema_upd) {   // fixed budget: update the row's EMA from the scores, then take its top-K'
      topk_row<kSRThreads, KPT, true>(scores + rr * N, const_cast<float*>(ema) + rr * N, alpha, first, N, Kp_next,
                                      pred_next + rr * Kp_next, nullptr, Force{0, N, sink, local});
      return;
    }
    if constexpr (KPT <= 16) {   // budgeted rows are routed elsewhere beyond 8192 blocks
      if (bp.policy != 0) {
        predict_row<kSRThreads, KPT, false>(scores + rr * N, const_cast<float*>(ema) + rr * N, 0.f, 0, N, Kp_next,
                                            bp, rr, pred_next + rr * Kp_next, Force{0, N, sink, local});
        return;
      }
    }
    topk_row<kSRThreads, KPT, false>(ema + rr * N, nullptr, 0.f, 0, N, Kp_next, pred_next + rr * Kp_next, nullptr,
                                     Force{0, N, sink, local});
    return;
  }
  topk_row<kSRThreads, KPT, false>(scores + r * N, nullptr, 0.f, 0, N, K, sel + r * K, s_T, Force{0, N, sink, local});

  // ---- T against P_t: slot of every entry of T in P_t (bisection when P_t is ascending) -------------------------
  const int b = (int)(r / Hkv), g = (int)(r % Hkv);
  const int32_t* prow = k_spec ? pred + r * k_spec : nullptr;
  if (tid == 0) { s_unsorted = 0; s_kf = k_spec; }
  for (int i = tid; i < k_spec; i += kSRThreads) s_P[i] = prow[i];
  __syncthreads();
  for (int i = tid; i < k_spec; i += kSRThreads)
    if (s_P[i] < 0) atomicMin(&s_kf, i);
  __syncthreads();
  const int kf = s_kf;   // the slots from the first empty one on never match
  for (int i = tid; i + 1 < kf; i += kSRThreads)
    if (s_P[i] >= s_P[i + 1]) s_unsorted = 1;
  __syncthreads();
  const bool sorted = s_unsorted == 0;
  constexpr int EPT = kSRMaxK / kSRThreads;   // entries per thread (4)
  int slot[EPT];
  uint32_t nh_local = 0;
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int j = tid * EPT + u;
    slot[u] = -1;
    if (j < K && kf > 0) {
      const int n = s_T[j];
      if (sorted) {
        int lo = 0, hi = kf;   // first index with s_P[idx] >= n
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_P[mid] < n) lo = mid + 1; else hi = mid;
        }
        if (lo < kf && s_P[lo] == n) slot[u] = lo;
      } else {
        for (int i = 0; i < kf; ++i)
          if (s_P[i] == n) { slot[u] = i; break; }
      }
    }
    nh_local += slot[u] >= 0;
  }
  uint32_t incl = nh_local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_scan[wave] = incl;
  __syncthreads();
  uint32_t before = 0, nh = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = s_scan[w];
    before += w < wave ? c : 0u;
    nh += c;
  }
  uint32_t ph = before + incl - nh_local;   // hits before this thread's entries
  int32_t* hrow = ws.hits + r * ws.Kp;
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int j = tid * EPT + u;
    if (j < K) {
      if (slot[u] >= 0) {
        hrow[ph] = slot[u];
        ++ph;
      } else {
        s_list[nh + (uint32_t)j - ph] = s_T[j];   // misses before entry j = j - hits before j
      }
    }
  }
  __syncthreads();
  const int nm = K - (int)nh;

  // ---- the missed blocks, shared among the waves, merged into one record --------------------------------------
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  const int m0 = (int)((int64_t)nm * wave / NW), m1 = (int)((int64_t)nm * (wave + 1) / NW);
  const int32_t* trow = table + (int64_t)b * pps;
  const int cap = 64 / ((bs + 15) >> 4);   // blocks per pipelined call
  for (int i0 = m0; i0 < m1; i0 += cap) {
    const int base = nh + i0;
    run_blocks<true>(st, min(cap, m1 - i0), [&](int i) { return s_list[base + i]; }, [](int) {}, kc, vc, trow, bs,
                     page, Hkv, g, N, last_len);
  }
  float folded[W::NK];
  st.fold(folded);
  st.store_ml(&s_ml[wave][0]);
#pragma unroll
  for (int i = 0; i < W::NK; ++i) {
    const int f = st.row * W::NK + i;
    s_o[wave][(f / W::VE) * D + st.col * W::VE + (f % W::VE)] = folded[i];
  }
  __syncthreads();
  float* rec = ws.mrec + r * (int64_t)RF;
  for (int f = tid; f < G * D; f += kSRThreads) {
    const int h = f / D;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h]);
    float o = 0.f;
    if (M > -__builtin_huge_valf()) {
#pragma unroll
      for (int w = 0; w < NW; ++w) o += s_o[w][f] * exp2f(s_ml[w][h] - M);
    }
    rec[ML + f] = o;
  }
  if (tid < G) {
    const int h = tid;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h]);
    float l = 0.f;
    if (M > -__builtin_huge_valf()) {
#pragma unroll
      for (int w = 0; w < NW; ++w) l += s_ml[w][G + h] * exp2f(s_ml[w][h] - M);
    }
    rec[h] = M;   // -inf and l = 0 when nothing was missed: the record then carries no weight
    rec[G + h] = l;
  }
  if (tid == 0) {
    ws.cnt[r] = (int)nh;
    n_missed[r] = nm;
  }
}

// out[b, g*G + h] = merge of the row's missed-block record and the speculated records of its hits, normalised. One
// 256-thread workgroup per (row, head): the weights exp2(m_i - M) go to LDS, then 256 / (D/4) record groups
// accumulate float4 slices of O with 8 loads in flight per thread.
template <int G, int D, int OB>
__global__ __launch_bounds__(256) void merge_hits_kernel(const float* __restrict__ partials, int k_spec, MissedWs ws,
                                                         float* __restrict__ out, int Hq, int Hkv) {
  constexpr int RF = rec_floats(G, D);
  constexpr int64_t SRB = spec_rec_bytes(OB == 4 ? 0 : 1, G, D);   // speculation record bytes
  constexpr int S = D / 4, P = 256 / S, U = 8;
  __shared__ float s_w[kSRMaxK + 1];
  __shared__ const uint8_t* s_rec[kSRMaxK + 1];
  __shared__ float s_red[2][4];
  __shared__ float4 s_acc[P][S];
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int b = (int)(r / Hkv), g = (int)(r % Hkv);
  const int nh = ws.cnt[r];
  const int n = nh + 1;   // record 0: the missed blocks; records 1..nh: speculated hits
  const uint8_t* mrec = reinterpret_cast<const uint8_t*>(ws.mrec + r * (int64_t)RF);
  const uint8_t* part_row = partials ? reinterpret_cast<const uint8_t*>(partials) + r * k_spec * SRB : nullptr;
  float mx = -__builtin_huge_valf();
  for (int i = t; i < n; i += 256) {   // record 0 (fp32 O) is the missed blocks', the rest speculated hits
    const uint8_t* rec = i == 0 ? mrec : part_row + (int64_t)ws.hits[r * ws.Kp + i - 1] * SRB;
    s_rec[i] = rec;
    const float m = reinterpret_cast<const float*>(rec)[h];
    s_w[i] = m;
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  float ls = 0.f;
  for (int i = t; i < n; i += 256) {
    const float w = exp2f(s_w[i] - M);
    s_w[i] = w;
    ls += reinterpret_cast<const float*>(s_rec[i])[G + h] * w;
  }
  ls = wave_sum(ls);
  if (lane == 0) s_red[1][wave] = ls;
  __syncthreads();
  const float L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  const int slot = t % S, p = t / S;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = p; i0 < n; i0 += U * P) {
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * P;
      o[u] = i < n ? rec_o4<G, D>(s_rec[i], OB == 4 || i == 0, h, slot) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * P;
      const float wr = i < n ? s_w[i] : 0.f;
      acc.x = fmaf(o[u].x, wr, acc.x); acc.y = fmaf(o[u].y, wr, acc.y);
      acc.z = fmaf(o[u].z, wr, acc.z); acc.w = fmaf(o[u].w, wr, acc.w);
    }
  }
  s_acc[p][slot] = acc;
  __syncthreads();
  if (t < S) {
    float4 a = s_acc[0][t];
#pragma unroll
    for (int p2 = 1; p2 < P; ++p2) {
      const float4 c = s_acc[p2][t];
      a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
    }
    const float il = 1.f / L;
    float* o = out + ((int64_t)b * Hq + (int64_t)g * G + h) * D;
    *reinterpret_cast<float4*>(o + t * 4) = make_float4(a.x * il, a.y * il, a.z * il, a.w * il);
  }
}

// ---- launchers -----------------------------------------------------------------------------------------------------

bool two_launch_supported(const prr_shape& s, int top_k, int k_spec, int k_spec_next) {
  return (s.page_size & 15) == 0 && s.block_size <= 128 && top_k <= kSRMaxK && k_spec <= kSRMaxK &&
         k_spec_next <= kSRMaxK && s.n_blocks <= 64 * kSRThreads;
}

template <int DT, int G>
static void score_spec_launch(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema,
                              float alpha, int first, const void* kc, const void* vc, const int32_t* table,
                              const int32_t* pred, int k_spec, float* partials, hipStream_t st) {
  const int rows = s.batch * s.n_kv_heads;
  const int chunk = score_chunk_size(s, ema != nullptr);
  const int gx = (s.n_blocks + chunk - 1) / chunk;
  const int spw = k_spec > 0 ? spec_slots_per_wave(s, k_spec) : 1;
  const int wpr = (k_spec + spw - 1) / spw;
  const int64_t spec_waves = (int64_t)rows * wpr;
  const int n_spec_wg = (int)((spec_waves + 3) / 4);
  const unsigned grid = (unsigned)(n_spec_wg + (int64_t)gx * rows);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* sm = static_cast<const uint8_t*>(summ);
  const auto* kk = static_cast<const uint8_t*>(kc);
  const auto* vv = static_cast<const uint8_t*>(vc);
  const float qs = s.softmax_scale * kLog2e;
  const bool p16 = (s.page_size & 15) == 0 && s.block_size <= 128;
#define PRR_SCORESPEC(EMA_, P16_)                                                                                   \
  score_spec_kernel<DT, G, EMA_, P16_><<<dim3(grid), dim3(256), 0, st>>>(                                          \
      qq, sm, scores, chunk, gx, ema, alpha, first, kk, vv, table, pred, k_spec, partials, n_spec_wg, spw, wpr,    \
      spec_waves, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size, s.pages_per_seq, qs,          \
      last_block_len(s), s.scorer)
  if (ema) {
    if (p16) PRR_SCORESPEC(true, true); else PRR_SCORESPEC(true, false);
  } else {
    if (p16) PRR_SCORESPEC(false, true); else PRR_SCORESPEC(false, false);
  }
#undef PRR_SCORESPEC
}

prr_status launch_score_spec(const prr_shape& s, const void* q, const void* summ, float* scores, float* ema,
                             float alpha, int first, const void* kc, const void* vc, const int32_t* table,
                             const int32_t* pred, int k_spec, float* partials, hipStream_t stream) {
  trace_begin(PRR_KERNEL_SCORE, stream);
  PRR_DISPATCH_DT_G(score_spec_launch, s, q, summ, scores, ema, alpha, first, kc, vc, table, pred, k_spec, partials,
                    stream);
  trace_end(PRR_KERNEL_SCORE, stream);
  return check_launch("score_speculate");
}

size_t select_missed_ws_bytes(const prr_shape& s, int top_k) {
  const int G = s.n_q_heads / s.n_kv_heads;
  return missed_ws_layout((int64_t)s.batch * s.n_kv_heads, top_k, (int)rec_floats(G, s.head_dim), nullptr, nullptr);
}

template <int DT, int G>
static void select_missed_launch(const prr_shape& s, const float* scores, int K, int32_t* sel, const float* ema,
                                 int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                                 const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                                 bool speculate, float* out, int32_t* n_missed, void* workspace, const BudgetDev& bp,
                                 hipStream_t st, bool ema_upd, float alpha, int first) {
  constexpr int D = 16 * Vec<DT>::n;
  const int rows = s.batch * s.n_kv_heads;
  MissedWs ws;
  missed_ws_layout(rows, K, (int)rec_floats(G, D), workspace, &ws);
  const int n_pwg = kp_next > 0 ? rows : 0;
  const int64_t spec_total = speculate ? (int64_t)rows * k_spec : 0;
  constexpr int WPG = kSRThreads / 64;
  const int n_spec_wg = (int)((spec_total + WPG - 1) / WPG);
  const dim3 grid((unsigned)(rows + n_pwg + n_spec_wg)), blk(kSRThreads);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* kk = static_cast<const uint8_t*>(kc);
  const auto* vv = static_cast<const uint8_t*>(vc);
  const float qs = s.softmax_scale * kLog2e;
#define PRR_SELMISS(KPT)                                                                                           \
  select_missed_kernel<KPT, DT, G><<<grid, blk, 0, st>>>(scores, K, sel, ema, kp_next, pred_next, qq, kk, vv,       \
                                                         table, pred, k_spec, partials, spec_total, ws, n_missed,   \
                                                         s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size,       \
                                                         s.page_size, s.pages_per_seq, qs, rows, n_pwg,             \
                                                         last_block_len(s), s.sink_blocks, s.local_blocks, bp,      \
                                                         ema_upd ? 1 : 0, alpha, first)
  trace_begin(PRR_KERNEL_SELECT_TOPK, st);
  if (s.n_blocks <= 4 * kSRThreads)
    PRR_SELMISS(4);
  else if (s.n_blocks <= 16 * kSRThreads)
    PRR_SELMISS(16);
  else
    PRR_SELMISS(64);
#undef PRR_SELMISS
  trace_end(PRR_KERNEL_SELECT_TOPK, st);
  trace_begin(PRR_KERNEL_FINALIZE, st);
  merge_hits_kernel<G, D, spec_o_bytes(DT)><<<dim3((unsigned)rows, (unsigned)G), dim3(256), 0, st>>>(
      partials, k_spec, ws, out, s.n_q_heads, s.n_kv_heads);
  trace_end(PRR_KERNEL_FINALIZE, st);
}

prr_status launch_select_missed(const prr_shape& s, const float* scores, int k, int32_t* sel, const float* ema,
                                int kp_next, int32_t* pred_next, const void* q, const void* kc, const void* vc,
                                const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                                bool speculate, float* out, int32_t* n_missed, void* workspace, hipStream_t stream,
                                const BudgetDev& bp, bool ema_upd, float alpha, int first) {
  if (ema_upd && (kp_next == 0 || !ema || bp.policy != 0)) {
    set_error("select_repair: the EMA update in the selection launch needs a predicted set of fixed size");
    return PRR_EINVAL;
  }
  PRR_DISPATCH_DT_G(select_missed_launch, s, scores, k, sel, ema, kp_next, pred_next, q, kc, vc, table, pred, k_spec,
                    partials, speculate, out, n_missed, workspace, bp, stream, ema_upd, alpha, first);
  return check_launch("select_repair");
}

}  // namespace prr
