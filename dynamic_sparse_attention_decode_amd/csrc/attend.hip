// Block-sparse decode attention: speculation over the predicted blocks, and repair-and-merge over the true set.
//
// PRR abstract: attention is speculated over the predicted blocks while selection is in flight; once the true set
// is known, the missed blocks are folded into the partial attention state with online-softmax statistics
// (FlashAttention-2, PRR reference list). PRR summary page (Key findings): full top-K coverage without
// recomputation, so the result is standard DSA over the true set.
//
// repair_kernel: grid (records per row, rows). Each wave walks `epw` consecutive entries of the true set T; an entry
// found in the predicted set P merges its speculated record, a missed entry is computed from the KV cache; entries
// of P outside T are never read. The 4 wave states merge in LDS into one record per workgroup.
// repair_row_kernel: one 8-wave workgroup per row where the rows fill the chip; T is split into hits and missed
// blocks first, the waves take even shares of both, and the workgroup writes the row's normalised output.
// finalize_kernel: one workgroup per (row, head) merges that head's part of the row's records, normalises, and
// writes out = O / l; the missed count is summed alongside.
#include "attn_wave.h"

namespace prr {

// One wave per `spw` consecutive predicted slots of one row (wpr waves per row).
template <int DT, int G, bool P16>
__global__ __launch_bounds__(256, 3) void speculate_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
                                                        const uint8_t* __restrict__ vc,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ pred, int k_spec,
                                                        float* __restrict__ partials, int Hq, int Hkv, int N, int bs,
                                                        int page, int pps, float qscale, int spw, int wpr,
                                                        int64_t total_waves, int last_len) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= total_waves) return;
  const int64_t rowid = w / wpr;
  const int j0 = (int)(w - rowid * wpr) * spw;
  const int j1 = min(k_spec, j0 + spw);
  speculate_slots<DT, G, P16>(rowid, j0, j1, threadIdx.x & 63, q, kc, vc, table, pred, k_spec, partials, Hq, Hkv, N, bs,
                              page, pps, qscale, last_len);
}

constexpr int kMaxRecords = 256;   // records per row (bounded through entries per wave)

// Merge one head's part of a row's records (m log2, l, O[D] of head h in every record), normalise, and write
// out[h][:]. One 256-thread workgroup: the n_rec (m, l) pairs are reduced with wave operations, then 256 / (D/4)
// record groups accumulate float4 slices of O with 8 loads in flight per thread.
template <int G, int D>
__device__ void finalize_head(const float* __restrict__ recs, int n_rec, int h, float* __restrict__ out_h) {
  constexpr int RF = rec_floats(G, D), ML = rec_ml(G);
  constexpr int S = D / 4;          // float4 slots of one head's O
  constexpr int P = 256 / S;        // record groups summed in parallel
  __shared__ float s_w[kMaxRecords];
  __shared__ float s_red[2][4];
  __shared__ float4 s_acc[P][S];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  // weights w_r = exp2(m_r - M) and L = sum_r l_r w_r
  const float mr = t < n_rec ? recs[(int64_t)t * RF + h] : -__builtin_huge_valf();
  const float lr = t < n_rec ? recs[(int64_t)t * RF + G + h] : 0.f;
  const float wm = wave_max(mr);
  if (lane == 0) s_red[0][wave] = wm;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float wgt = t < n_rec ? exp2f(mr - M) : 0.f;
  s_w[t] = wgt;
  const float ls = wave_sum(lr * wgt);
  if (lane == 0) s_red[1][wave] = ls;
  __syncthreads();
  const float L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  const int slot = t % S, p = t / S;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int U = 8;
  for (int r0 = p; r0 < n_rec; r0 += U * P) {
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * P;
      o[u] = r < n_rec ? *reinterpret_cast<const float4*>(recs + (int64_t)r * RF + ML + h * D + slot * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * P;
      const float wr = r < n_rec ? s_w[r] : 0.f;
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
    *reinterpret_cast<float4*>(out_h + t * 4) = make_float4(a.x * il, a.y * il, a.z * il, a.w * il);
  }
}

// Two workgroups per CU from G = 4 up: three (168 VGPRs) spilled a register at G = 4 (same-box A/B over two runs:
// 32K layer PRR step 20.80 -> 20.41 us, serialized 19.95 -> 19.64 us; 131K batch 45.9 -> 45.1 and 33.7 -> 33.5 us).
template <int DT, int G, bool P16>
__global__ __launch_bounds__(256, G >= 4 ? 2 : 3) void repair_kernel(const uint8_t* __restrict__ q,
                                                     const uint8_t* __restrict__ kc,
                                                     const uint8_t* __restrict__ vc,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ sel, int top_k,
                                                     const int32_t* __restrict__ pred, int k_spec,
                                                     const float* __restrict__ partials, float* __restrict__ ws_rec,
                                                     int32_t* __restrict__ ws_miss, int Hq, int Hkv, int N, int bs,
                                                     int page, int pps, float qscale, int epw, int last_len) {
  using W = Tile<DT, G>;
  constexpr int NW = 4, NT = NW * 64;
  constexpr int D = W::D;
  constexpr int RF = rec_floats(G, D);
  constexpr int ML = rec_ml(G);
  constexpr int kPredLds = 2048;   // predicted sets up to this size are searched in LDS
  __shared__ float s_ml[NW][2 * G];
  __shared__ float s_o[NW * G * D];
  __shared__ int s_miss[NW];
  __shared__ int32_t s_pred[kPredLds];
  __shared__ int32_t s_mid[NW][8];   // missed block ids of the current group of entries, per wave
  __shared__ int s_kf[NW];           // per wave: the first empty (negative) slot of P it saw
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rowid = blockIdx.y;
  const int rec = blockIdx.x;
  const int n_rec = gridDim.x;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int32_t* srow = sel + rowid * top_k;
  const int32_t* prow = pred ? pred + rowid * k_spec : nullptr;
  const uint8_t* part_row =
      partials ? reinterpret_cast<const uint8_t*>(partials) + rowid * k_spec * W::kSpecRecBytes : nullptr;

  const bool pred_lds = k_spec <= kPredLds;
  int kneg = k_spec;
  if (prow)
    for (int i = threadIdx.x; i < k_spec; i += NT) {
      const int32_t v = prow[i];
      if (pred_lds) s_pred[i] = v;
      if (v < 0) kneg = min(kneg, i);
    }
  kneg = -(int)wave_max(-(float)kneg);   // exact: slot counts are far below 2^24
  if (lane == 0) s_kf[wave] = kneg;
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  const int32_t* trow = table + (int64_t)b * pps;
  __syncthreads();
  // slots from the first empty one on never match (speculation may have skipped them), as in the row-wise repair
  int kf = s_kf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) kf = min(kf, s_kf[w]);
  int misses = 0;
  const int j0 = (rec * NW + wave) * epw;
  const int j1 = min(top_k, j0 + epw);
  for (int jb = j0; jb < j1; jb += 8) {
    // look up up to 8 entries: merge the speculated ones, collect the missed ones
    int nm = 0;
    for (int j = jb; j < min(j1, jb + 8); ++j) {
      const int n = min(max(srow[j], 0), N - 1);
      int slot = -1;
      for (int c = 0; c < kf; c += 64) {
        const int i = c + lane;
        const int pv = i < kf ? (pred_lds ? s_pred[i] : prow[i]) : -1;
        const unsigned long long hit = __ballot(pv == n);
        if (hit) { slot = c + __ffsll(hit) - 1; break; }
      }
      if (slot >= 0) {
        st.merge_spec_record(part_row + (int64_t)slot * W::kSpecRecBytes);
      } else {
        if (lane == 0) s_mid[wave][nm] = n;
        ++nm;
      }
    }
    misses += nm;
    // compute the missed blocks with the next chunk's loads in flight
    run_blocks<P16>(st, nm, [&](int i) { return s_mid[wave][i]; }, [](int) {}, kc, vc, trow, bs, page, Hkv, g, N,
                    last_len);
  }
  float folded[W::NK];
  st.fold(folded);
  st.store_ml(&s_ml[wave][0]);
  if (lane == 0) s_miss[wave] = misses;
#pragma unroll
  for (int i = 0; i < W::NK; ++i) {
    const int f = st.row * W::NK + i;
    s_o[wave * G * D + (f / W::VE) * D + st.col * W::VE + (f % W::VE)] = folded[i];
  }
  __syncthreads();
  // merge the wave states into this workgroup's record
  float* my = ws_rec + (rowid * n_rec + rec) * (int64_t)RF;
  for (int f = threadIdx.x; f < G * D; f += NT) {
    const int h = f / D;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += s_o[w * G * D + f] * exp2f(s_ml[w][h] - M);
    my[ML + f] = o;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += s_ml[w][G + h] * exp2f(s_ml[w][h] - M);
    my[h] = M;
    my[G + h] = L;
  }
  if (threadIdx.x == 0) {
    int m = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) m += s_miss[w];
    ws_miss[rowid * n_rec + rec] = m;
  }
}

// One 8-wave workgroup per row (K <= kRowMaxK): the row's true set T is looked up in the predicted set P once, by
// one thread per entry (bisection when P is ascending, as the selection writes it; a linear search otherwise), and
// split into a list of the hits' slots and a list of the missed blocks with a workgroup prefix count. Each wave then
// takes an even share of the missed blocks (one pipelined run) and of the hits (record merges), so no wave carries
// more than its share of either; the wave states merge in LDS into the row's normalised output.
constexpr int kRowMaxK = 128;

template <int DT, int G, bool P16>
__global__ __launch_bounds__(512, 1) void repair_row_kernel(const uint8_t* __restrict__ q,
                                                            const uint8_t* __restrict__ kc,
                                                            const uint8_t* __restrict__ vc,
                                                            const int32_t* __restrict__ table,
                                                            const int32_t* __restrict__ sel, int top_k,
                                                            const int32_t* __restrict__ pred, int k_spec,
                                                            const float* __restrict__ partials, int Hq, int Hkv,
                                                            int N, int bs, int page, int pps, float qscale,
                                                            int last_len, float* __restrict__ out,
                                                            int32_t* __restrict__ n_missed) {
  using W = Tile<DT, G>;
  constexpr int NW = 8, NT = 512;
  constexpr int D = W::D;
  constexpr int kPredLds = 2048;
  __shared__ float s_ml[NW][2 * G];
  __shared__ float s_o[NW * G * D];
  __shared__ int32_t s_pred[kPredLds];
  __shared__ int32_t s_hit[kRowMaxK];   // predicted slots of the hits, in T order
  __shared__ int32_t s_mid[kRowMaxK];   // missed block ids, in T order
  __shared__ int s_cnt[2][2];           // per half of T (waves 0 and 1): hits in it
  __shared__ int s_kf, s_unsorted;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t rowid = blockIdx.x;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int32_t* srow = sel + rowid * top_k;
  const int32_t* prow = pred ? pred + rowid * k_spec : nullptr;
  const uint8_t* part_row =
      partials ? reinterpret_cast<const uint8_t*>(partials) + rowid * k_spec * W::kSpecRecBytes : nullptr;
  const bool pred_lds = k_spec <= kPredLds;
  if (t == 0) { s_kf = prow ? k_spec : 0; s_unsorted = 0; }
  __syncthreads();
  if (prow)
    for (int i = t; i < k_spec; i += NT) {
      const int32_t v = prow[i];
      if (pred_lds) s_pred[i] = v;
      if (v < 0) atomicMin(&s_kf, i);
    }
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  const int32_t* trow = table + (int64_t)b * pps;
  __syncthreads();
  // slots from the first empty one on never match (speculation may have skipped them)
  const int kf = s_kf;
  if (pred_lds)
    for (int i = t; i + 1 < kf; i += NT)
      if (s_pred[i] >= s_pred[i + 1]) s_unsorted = 1;
  __syncthreads();
  const bool sorted = pred_lds && s_unsorted == 0;
  // one thread per entry of T (threads 0 .. K-1 are waves 0 and 1)
  int n = 0, slot = -1;
  if (t < top_k) {
    n = min(max(srow[t], 0), N - 1);
    if (sorted) {
      int lo = 0, hi = kf;   // first index with s_pred[idx] >= n
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_pred[mid] < n) lo = mid + 1; else hi = mid;
      }
      if (lo < kf && s_pred[lo] == n) slot = lo;
    } else {
      for (int i = 0; i < kf; ++i)
        if ((pred_lds ? s_pred[i] : prow[i]) == n) { slot = i; break; }
    }
  }
  const unsigned long long hm = __ballot(t < top_k && slot >= 0);
  const unsigned long long vm = __ballot(t < top_k);
  if (wave < 2 && lane == 0) { s_cnt[wave][0] = __popcll(hm); s_cnt[wave][1] = __popcll(vm & ~hm); }
  __syncthreads();
  const int nh = s_cnt[0][0] + s_cnt[1][0], nm = s_cnt[0][1] + s_cnt[1][1];
  if (t < top_k) {
    const unsigned long long below = (1ull << lane) - 1ull;
    const int hb = (wave == 1 ? s_cnt[0][0] : 0) + __popcll(hm & below);
    const int mb = (wave == 1 ? s_cnt[0][1] : 0) + __popcll(vm & ~hm & below);
    if (slot >= 0) s_hit[hb] = slot; else s_mid[mb] = n;
  }
  __syncthreads();
  // even shares: missed blocks [m0, m1) and hits [h0, h1) of this wave
  const int m0 = wave * nm / NW, m1 = (wave + 1) * nm / NW;
  const int h0 = wave * nh / NW, h1 = (wave + 1) * nh / NW;
  constexpr int kRun = 8;   // missed blocks per pipelined run (at most 64 chunks)
  for (int mb = m0; mb < m1; mb += kRun)
    run_blocks<P16>(st, min(kRun, m1 - mb), [&](int i) { return s_mid[mb + i]; }, [](int) {}, kc, vc, trow, bs,
                    page, Hkv, g, N, last_len);
  for (int i = h0; i < h1; ++i) st.merge_spec_record(part_row + (int64_t)s_hit[i] * W::kSpecRecBytes);
  float folded[W::NK];
  st.fold(folded);
  st.store_ml(&s_ml[wave][0]);
#pragma unroll
  for (int i = 0; i < W::NK; ++i) {
    const int f = st.row * W::NK + i;
    s_o[wave * G * D + (f / W::VE) * D + st.col * W::VE + (f % W::VE)] = folded[i];
  }
  __syncthreads();
  for (int f = t; f < G * D; f += NT) {
    const int h = f / D;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = exp2f(s_ml[w][h] - M);
      o += s_o[w * G * D + f] * c;
      L += s_ml[w][G + h] * c;
    }
    out[((int64_t)b * Hq + (int64_t)g * G) * D + f] = o / L;
  }
  if (t == 0) n_missed[rowid] = nm;
}

// Merge each row's records into the normalised output: one workgroup per (row, head); the head-0 workgroup also sums
// the missed count. A kernel boundary separates it from repair_kernel: publishing each workgroup's record with an
// agent-scope release fence (an L2 write-back on this multi-XCD part; the fences serialise) costs about 5.5 us over
// 256 workgroups, against 1.6-2.1 us for a launch in a graph.
template <int G, int D>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ ws_rec,
                                                       const int32_t* __restrict__ ws_miss, int n_rec,
                                                       float* __restrict__ out, int32_t* __restrict__ n_missed,
                                                       int Hq, int Hkv) {
  const int64_t rowid = blockIdx.x;
  const int h = blockIdx.y;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  finalize_head<G, D>(ws_rec + rowid * n_rec * rec_floats(G, D), n_rec, h,
                      out + ((int64_t)b * Hq + (int64_t)g * G + h) * D);
  if (h == 0 && threadIdx.x < 64) {
    int c = 0;
    for (int r = threadIdx.x; r < n_rec; r += 64) c += ws_miss[rowid * n_rec + r];
    c = (int)wave_sum((float)c);   // exact: counts are far below 2^24
    if (threadIdx.x == 0) n_missed[rowid] = c;
  }
}

// ---- launchers -----------------------------------------------------------------------------------------------------

// Entries of T per repair wave: enough to keep records per row <= kMaxRecords; on the pipelined path about eight
// 16-token chunks per wave while at least 4096 waves remain (on the paged batch, 8 entries per wave against 4:
// repair 57.5 -> 53.8 us, 4 against 2: 62.1 -> 57.0 us), and sixteen one-chunk entries where eight would leave that
// many waves: every workgroup is then resident at once, which the PRR step's mix of record merges and missed blocks
// needs (paged batch, same-box A/B over three runs: PRR step 215.8 -> 213.1 us; serialized 147.8 -> 147.6 us).
static int repair_epw(const prr_shape& s, int top_k) {
  const int need = (top_k + 4 * kMaxRecords - 1) / (4 * kMaxRecords);
  int e = 1;
  if ((s.page_size & 15) == 0 && s.block_size <= 128) {
    const int cpb = (s.block_size + 15) / 16;
    e = cpb >= 8 ? 1 : 8 / cpb;
    const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
    while (e > 1 && rows * ((top_k + e - 1) / e) < 4096) e >>= 1;
    if (cpb == 1 && e == 8) e = 16;
  }
  return e > need ? e : need;
}

static int repair_records(const prr_shape& s, int top_k) {
  const int per = 4 * repair_epw(s, top_k);
  return (top_k + per - 1) / per;
}

struct RepairWs {
  float* rec;
  int32_t* miss;
};

static size_t ws_layout(const prr_shape& s, int top_k, void* base, RepairWs* out) {
  const int G = s.n_q_heads / s.n_kv_heads;
  const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
  const int64_t nrec = repair_records(s, top_k);
  const size_t rec_bytes = (size_t)(rows * nrec * rec_floats(G, s.head_dim)) * sizeof(float);
  const size_t miss_bytes = ((size_t)(rows * nrec) * sizeof(int32_t) + 255) / 256 * 256;
  if (out) {
    char* p = static_cast<char*>(base);
    out->rec = reinterpret_cast<float*>(p);
    out->miss = reinterpret_cast<int32_t*>(p + rec_bytes);
  }
  return rec_bytes + miss_bytes;
}

size_t repair_workspace_bytes(const prr_shape& s, int top_k) { return ws_layout(s, top_k, nullptr, nullptr); }

// The resolved-page pipelined path: 16-token chunks never straddle a page, and a wave's group of at most 8 entries
// (or 4 speculation slots) spans at most 64 chunks.
bool p16_path(const prr_shape& s) { return (s.page_size & 15) == 0 && s.block_size <= 128; }

// Slots per speculation wave: about four 16-token chunks per wave, while keeping at least 4096 waves in flight.
int spec_slots_per_wave(const prr_shape& s, int k_spec) {
  const int cpb = (s.block_size + 15) / 16;
  int spw = cpb >= 4 ? 1 : 4 / cpb;
  const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
  while (spw > 1 && rows * ((k_spec + spw - 1) / spw) < 4096) spw >>= 1;
  return spw;
}

template <int DT, int G>
static void spec_launch(const prr_shape& s, const void* q, const void* kc, const void* vc, const int32_t* table,
                        const int32_t* pred, int k_spec, float* partials, hipStream_t st) {
  const int spw = spec_slots_per_wave(s, k_spec);
  const int wpr = (k_spec + spw - 1) / spw;
  const int64_t total = (int64_t)s.batch * s.n_kv_heads * wpr;
  const float qscale = s.softmax_scale * kLog2e;
  trace_begin(PRR_KERNEL_SPECULATE, st);
  auto kern = p16_path(s) ? speculate_kernel<DT, G, true> : speculate_kernel<DT, G, false>;
  kern<<<dim3((unsigned)((total + 3) / 4)), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, pred,
      k_spec, partials, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size, s.pages_per_seq, qscale,
      spw, wpr, total, last_block_len(s));
  trace_end(PRR_KERNEL_SPECULATE, st);
}

// One 8-wave workgroup per row that writes the output itself (no merge launch) where the row's true set fits it and
// the rows alone fill the chip: one workgroup per CU at these register counts (paged batch, same-box A/B: with the
// wave-per-16-entries split 210.1 -> 203.5 us, with even shares of the hits and the missed blocks 203.3 -> 199.0).
static bool repair_row_wg(const prr_shape& s, int top_k, int epw) {
  return (int64_t)s.batch * s.n_kv_heads >= 256 && top_k <= 8 * epw && top_k <= kRowMaxK;
}

template <int DT, int G>
static void repair_launch(const prr_shape& s, const void* q, const void* kc, const void* vc, const int32_t* table,
                          const int32_t* sel, int top_k, const int32_t* pred, int k_spec, const float* partials,
                          float* out, int32_t* n_missed, void* workspace, hipStream_t st) {
  const int epw = repair_epw(s, top_k);
  const int nrec = repair_records(s, top_k);
  const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
  RepairWs ws;
  ws_layout(s, top_k, workspace, &ws);
  const float qscale = s.softmax_scale * kLog2e;
  const bool p16 = p16_path(s);
  if (repair_row_wg(s, top_k, epw)) {
    trace_begin(PRR_KERNEL_REPAIR, st);
    auto kern = p16 ? repair_row_kernel<DT, G, true> : repair_row_kernel<DT, G, false>;
    kern<<<dim3((unsigned)rows), dim3(512), 0, st>>>(
        static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, sel,
        top_k, pred, k_spec, partials, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size,
        s.pages_per_seq, qscale, last_block_len(s), out, n_missed);
    trace_end(PRR_KERNEL_REPAIR, st);
    return;
  }
  trace_begin(PRR_KERNEL_REPAIR, st);
  auto kern = p16 ? repair_kernel<DT, G, true> : repair_kernel<DT, G, false>;
  kern<<<dim3((unsigned)nrec, (unsigned)rows), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, sel,
      top_k, pred, k_spec, partials, ws.rec, ws.miss, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size,
      s.page_size, s.pages_per_seq, qscale, epw, last_block_len(s));
  trace_end(PRR_KERNEL_REPAIR, st);
  constexpr int D = 16 * Vec<DT>::n;
  trace_begin(PRR_KERNEL_FINALIZE, st);
  finalize_kernel<G, D><<<dim3((unsigned)rows, (unsigned)G), dim3(256), 0, st>>>(ws.rec, ws.miss, nrec, out,
                                                                                 n_missed, s.n_q_heads,
                                                                                 s.n_kv_heads);
  trace_end(PRR_KERNEL_FINALIZE, st);
}

prr_status launch_speculate(const prr_shape& s, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* table, const int32_t* pred, int k_spec, float* partials,
                            hipStream_t stream) {
  if (k_spec == 0) return PRR_OK;
  PRR_DISPATCH_DT_G(spec_launch, s, q, k_cache, v_cache, table, pred, k_spec, partials, stream);
  return check_launch("speculate");
}

prr_status launch_repair(const prr_shape& s, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* table, const int32_t* sel, int top_k, const int32_t* pred, int k_spec,
                         const float* partials, float* out, int32_t* n_missed, void* workspace, hipStream_t stream) {
  if (!pred || !partials) k_spec = 0;
  PRR_DISPATCH_DT_G(repair_launch, s, q, k_cache, v_cache, table, sel, top_k, pred, k_spec, partials, out, n_missed,
                    workspace, stream);
  return check_launch("repair_merge");
}

}  // namespace prr
