// Block-sparse decode attention: speculation over the predicted blocks, and repair-and-merge over the true set.
//
// PRR abstract: attention is speculated over the predicted blocks while selection is in flight; once the true set
// is known, the missed blocks are folded into the partial attention state with online-softmax statistics
// (FlashAttention-2, PRR reference list). PRR summary page (Key findings): full top-K coverage without
// recomputation, so the result is standard DSA over the true set.
//
// Work unit: one wave processes one (sequence b, KV head g, block) for all G query heads of the group. Each load
// instruction reads 4 token rows of K (16 lanes x 16 B per 256-byte row, lane = 16*row + col) and the same 4 rows
// of V, coalesced, through the paged block table. Per token the group's G logits are full 16-lane DPP sums; the
// running max is kept uniform across the wave, while l and the O accumulator stay per-lane partial sums over the
// lane's token rows until the end, when two permlane swaps fold the 4 rows (each lane then owns G*VE/4 outputs).
// Logits are kept in log2 units (q pre-scaled by softmax_scale * log2 e) so every exponential is one exp2.
//
// Partial record (per (b, g, slot)): m[G] (log2 units), l[G], zero padding to a multiple of 4 floats, then O[G][D]
// (unnormalised), fp32; records are 16-byte aligned.
#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

template <int DT, int G>
struct AttnWave {
  using V = Vec<DT>;
  static constexpr int VE = V::n;       // elements per 16-byte load
  static constexpr int D = 16 * VE;     // head_dim
  static constexpr int NV = G * VE;     // accumulator values per lane
  static constexpr int NK = NV / 4;     // values per lane after folding the 4 rows
  static constexpr int ML = rec_ml(G);  // offset of O in a record (floats)

  float q[G][VE];
  float m[G];      // running max, log2 units, uniform across the wave
  float l[G];      // per-lane partial sum over this lane's token rows
  float acc[G][VE];
  int lane, row, col;

  __device__ void init(int lane_) {
    lane = lane_;
    row = lane >> 4;
    col = lane & 15;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -__builtin_huge_valf();
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;
    }
  }

  __device__ void load_q(const uint8_t* qg, float qscale) {   // qg = q + (b*Hq + g*G) * 256
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x[VE];
      V::to_f32(ld16(qg + h * kRowBytes + col * 16), x);
#pragma unroll
      for (int e = 0; e < VE; ++e) q[h][e] = x[e] * qscale;
    }
  }

  // Fold one block of bs tokens (bs % 4 == 0) into the running state.
  __device__ void block(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                        const int32_t* __restrict__ trow, int n, int bs, int page, int Hkv, int g) {
    const int64_t tok0 = (int64_t)n * bs;
    for (int t0 = 0; t0 < bs; t0 += 16) {
      uint4 kv[4], vv[4];
      bool ok[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[j] = t0 + 4 * j < bs;
        const int64_t tok = tok0 + t0 + 4 * j + row;
        if (ok[j]) {
          const int64_t phys = trow[tok / page];
          const int64_t off = ((phys * Hkv + g) * page + tok % page) * (int64_t)kRowBytes + col * 16;
          kv[j] = ld16(kc + off);
          vv[j] = ld16(vc + off);
        } else {
          kv[j] = make_uint4(0, 0, 0, 0);
          vv[j] = make_uint4(0, 0, 0, 0);
        }
      }
      float z[4][G];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x[VE];
        V::to_f32(kv[j], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) s = fmaf(q[h][e], x[e], s);
          s = row_sum16(s);
          z[j][h] = ok[j] ? s : -__builtin_huge_valf();
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mc = fmaxf(fmaxf(z[0][h], z[1][h]), fmaxf(z[2][h], z[3][h]));
        mc = max_xor32(max_xor16(mc));
        const float mn = fmaxf(m[h], mc);
        const float corr = exp2f(m[h] - mn);
        m[h] = mn;
        l[h] *= corr;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] *= corr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[j][h] = exp2f(z[j][h] - mn);
          l[h] += z[j][h];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[VE];
        V::to_f32(vv[j], y);
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[h][e] = fmaf(z[j][h], y[e], acc[h][e]);
        }
      }
    }
  }

  // Merge a stored partial record (m[G] log2, l[G], O[G][D]) into the running state. The record's l and O are
  // added by one row only (row h % 4), since the rows are summed when the state is folded.
  __device__ void merge_record(const float* __restrict__ rec) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mr = rec[h];
      const float lr = rec[G + h];
      const float mn = fmaxf(m[h], mr);
      const float c_old = exp2f(m[h] - mn);
      const float c_new = exp2f(mr - mn);
      m[h] = mn;
      const bool mine = row == (h & 3);
      l[h] = l[h] * c_old + (mine ? lr * c_new : 0.f);
      float o[VE] = {};
      if (mine) {
        const float* src = rec + ML + h * D + col * VE;
#pragma unroll
        for (int e = 0; e < VE; e += 4) {
          const float4 t = *reinterpret_cast<const float4*>(src + e);
          o[e] = t.x; o[e + 1] = t.y; o[e + 2] = t.z; o[e + 3] = t.w;
        }
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[h][e] = acc[h][e] * c_old + (mine ? o[e] * c_new : 0.f);
    }
  }

  // Fold the 4 rows: l becomes the wave total (uniform); out[i] holds flat accumulator f = row*NK + i.
  __device__ void fold(float* out) {
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = sum_xor32(sum_xor16(l[h]));
    float t[NV / 2];
#pragma unroll
    for (int f = 0; f < NV / 2; ++f) {
      const int f2 = f + NV / 2;
      t[f] = fold32(acc[f / VE][f % VE], acc[f2 / VE][f2 % VE]);
    }
#pragma unroll
    for (int f = 0; f < NK; ++f) out[f] = fold16(t[f], t[f + NK]);
  }

  // Write the folded state as a record.
  __device__ void write_record(float* __restrict__ rec, const float* folded) {
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) { rec[h] = m[h]; rec[G + h] = l[h]; }
    }
    float* o = rec + ML;
    if constexpr (NK % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NK; i += 4) {
        const int f = row * NK + i;
        const int h = f / VE, e = f % VE;
        *reinterpret_cast<float4*>(o + h * D + col * VE + e) =
            make_float4(folded[i], folded[i + 1], folded[i + 2], folded[i + 3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int f = row * NK + i;
        o[(f / VE) * D + col * VE + (f % VE)] = folded[i];
      }
    }
  }
};

// ---- speculation: one record per predicted slot ----------------------------------------------------------------

template <int DT, int G>
__global__ __launch_bounds__(256) void speculate_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
                                                        const uint8_t* __restrict__ vc,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ pred, int k_spec,
                                                        float* __restrict__ partials, int Hq, int Hkv, int N, int bs,
                                                        int page, int pps, float qscale, int64_t total) {
  using W = AttnWave<DT, G>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + wave;
  if (s >= total) return;
  const int64_t rowid = s / k_spec;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int n = min(max(pred[s], 0), N - 1);   // ids outside [0, N) are clamped: wrong output, never a fault
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  st.block(kc, vc, table + (int64_t)b * pps, n, bs, page, Hkv, g);
  float folded[W::NK];
  st.fold(folded);
  st.write_record(partials + s * rec_floats(G, W::D), folded);
}

// ---- repair: per workgroup a slice of the true set; hits reuse speculated records, misses are computed --------

template <int DT, int G>
__global__ __launch_bounds__(256) void repair_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
                                                     const uint8_t* __restrict__ vc,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ sel, int top_k,
                                                     const int32_t* __restrict__ pred, int k_spec,
                                                     const float* __restrict__ partials,
                                                     float* __restrict__ ws_rec, int32_t* __restrict__ ws_miss,
                                                     int Hq, int Hkv, int N, int bs, int page, int pps,
                                                     float qscale, int epw) {
  using W = AttnWave<DT, G>;
  constexpr int RF = rec_floats(G, W::D);
  constexpr int ML = rec_ml(G);
  __shared__ float s_ml[4][2 * G];
  __shared__ float s_o[4][G * W::D];
  __shared__ int s_miss[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rowid = blockIdx.y;
  const int rec = blockIdx.x;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int32_t* srow = sel + rowid * top_k;
  const int32_t* prow = pred ? pred + rowid * k_spec : nullptr;
  const float* part_row = partials ? partials + rowid * k_spec * (int64_t)RF : nullptr;

  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  const int32_t* trow = table + (int64_t)b * pps;
  int misses = 0;
  const int j0 = (rec * 4 + wave) * epw;
  const int j1 = min(top_k, j0 + epw);
  for (int j = j0; j < j1; ++j) {
    const int n = min(max(srow[j], 0), N - 1);
    int slot = -1;
    for (int c = 0; c < k_spec; c += 64) {
      const int i = c + lane;
      const int pv = i < k_spec ? prow[i] : -1;
      const unsigned long long hit = __ballot(pv == n);
      if (hit) { slot = c + __ffsll(hit) - 1; break; }
    }
    if (slot >= 0) {
      st.merge_record(part_row + (int64_t)slot * RF);
    } else {
      st.block(kc, vc, trow, n, bs, page, Hkv, g);
      ++misses;
    }
  }
  float folded[W::NK];
  st.fold(folded);
  // per-wave state to LDS
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_ml[wave][h] = st.m[h]; s_ml[wave][G + h] = st.l[h]; }
    s_miss[wave] = misses;
  }
#pragma unroll
  for (int i = 0; i < W::NK; ++i) {
    const int f = st.row * W::NK + i;
    s_o[wave][(f / W::VE) * W::D + st.col * W::VE + (f % W::VE)] = folded[i];
  }
  __syncthreads();
  // workgroup merge of the 4 wave states into one record
  float* out = ws_rec + (rowid * gridDim.x + rec) * (int64_t)RF;
  for (int f = threadIdx.x; f < G * W::D; f += 256) {
    const int h = f / W::D;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_ml[w][h]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o += s_o[w][f] * exp2f(s_ml[w][h] - M);
    out[ML + f] = o;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = s_ml[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_ml[w][h]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += s_ml[w][G + h] * exp2f(s_ml[w][h] - M);
    out[h] = M;
    out[G + h] = L;
  }
  if (threadIdx.x == 0) ws_miss[rowid * gridDim.x + rec] = s_miss[0] + s_miss[1] + s_miss[2] + s_miss[3];
}

// ---- final merge of the slice records and normalisation ------------------------------------------------------

template <int G, int D>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ ws_rec,
                                                       const int32_t* __restrict__ ws_miss, int n_rec,
                                                       float* __restrict__ out, int32_t* __restrict__ n_missed,
                                                       int Hq, int Hkv) {
  constexpr int RF = rec_floats(G, D);
  constexpr int ML = rec_ml(G);
  __shared__ float s_M[G], s_L[G];
  __shared__ float red[256];
  const int64_t rowid = blockIdx.x;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const float* recs = ws_rec + rowid * n_rec * (int64_t)RF;
  const int t = threadIdx.x;
  // per-head maximum and rescaled sum over the records
  for (int h = 0; h < G; ++h) {
    float M = -__builtin_huge_valf();
    for (int r = t; r < n_rec; r += 256) M = fmaxf(M, recs[(int64_t)r * RF + h]);
    red[t] = M;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) red[t] = fmaxf(red[t], red[t + s]);
      __syncthreads();
    }
    M = red[0];
    __syncthreads();
    float L = 0.f;
    for (int r = t; r < n_rec; r += 256) L += recs[(int64_t)r * RF + G + h] * exp2f(recs[(int64_t)r * RF + h] - M);
    red[t] = L;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) red[t] += red[t + s];
      __syncthreads();
    }
    if (t == 0) { s_M[h] = M; s_L[h] = red[0]; }
    __syncthreads();
  }
  for (int f = t; f < G * D; f += 256) {
    const int h = f / D;
    const float M = s_M[h];
    float o = 0.f;
    for (int r = 0; r < n_rec; ++r) o += recs[(int64_t)r * RF + ML + f] * exp2f(recs[(int64_t)r * RF + h] - M);
    out[((int64_t)b * Hq + (int64_t)g * G + h) * D + (f % D)] = o / s_L[h];
  }
  if (t == 0) {
    int s = 0;
    for (int r = 0; r < n_rec; ++r) s += ws_miss[rowid * n_rec + r];
    n_missed[rowid] = s;
  }
}

// ---- launchers -----------------------------------------------------------------------------------------------------

static int repair_epw(const prr_shape& s, int top_k) {
  const int64_t entries = (int64_t)s.batch * s.n_kv_heads * top_k;
  return entries > 16384 ? 2 : 1;
}

static int repair_records(const prr_shape& s, int top_k) {
  const int per = 4 * repair_epw(s, top_k);
  return (top_k + per - 1) / per;
}

size_t repair_workspace_bytes(const prr_shape& s, int top_k) {
  const int G = s.n_q_heads / s.n_kv_heads;
  const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
  const int64_t nrec = repair_records(s, top_k);
  const size_t rec_bytes = (size_t)(rows * nrec * rec_floats(G, s.head_dim)) * sizeof(float);
  return rec_bytes + (size_t)(rows * nrec) * sizeof(int32_t) + 256;
}

template <int DT, int G>
static void spec_launch(const prr_shape& s, const void* q, const void* kc, const void* vc, const int32_t* table,
                        const int32_t* pred, int k_spec, float* partials, hipStream_t st) {
  const int64_t total = (int64_t)s.batch * s.n_kv_heads * k_spec;
  const float qscale = s.softmax_scale * kLog2e;
  trace_begin(PRR_KERNEL_SPECULATE, st);
  speculate_kernel<DT, G><<<dim3((unsigned)((total + 3) / 4)), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, pred,
      k_spec, partials, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size, s.page_size, s.pages_per_seq, qscale,
      total);
  trace_end(PRR_KERNEL_SPECULATE, st);
}

template <int DT, int G>
static void repair_launch(const prr_shape& s, const void* q, const void* kc, const void* vc, const int32_t* table,
                          const int32_t* sel, int top_k, const int32_t* pred, int k_spec, const float* partials,
                          float* out, int32_t* n_missed, void* workspace, hipStream_t st) {
  constexpr int D = 16 * Vec<DT>::n;
  const int epw = repair_epw(s, top_k);
  const int nrec = repair_records(s, top_k);
  const int64_t rows = (int64_t)s.batch * s.n_kv_heads;
  auto* ws_rec = static_cast<float*>(workspace);
  auto* ws_miss = reinterpret_cast<int32_t*>(ws_rec + rows * nrec * rec_floats(G, D));
  const float qscale = s.softmax_scale * kLog2e;
  trace_begin(PRR_KERNEL_REPAIR, st);
  repair_kernel<DT, G><<<dim3((unsigned)nrec, (unsigned)rows), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), table, sel,
      top_k, pred, k_spec, partials, ws_rec, ws_miss, s.n_q_heads, s.n_kv_heads, s.n_blocks, s.block_size,
      s.page_size, s.pages_per_seq, qscale, epw);
  trace_end(PRR_KERNEL_REPAIR, st);
  trace_begin(PRR_KERNEL_FINALIZE, st);
  finalize_kernel<G, D><<<dim3((unsigned)rows), dim3(256), 0, st>>>(ws_rec, ws_miss, nrec, out, n_missed,
                                                                    s.n_q_heads, s.n_kv_heads);
  trace_end(PRR_KERNEL_FINALIZE, st);
}

#define PRR_DISPATCH_DT_G(FN, ...)                                      \
  do {                                                                  \
    const int G_ = s.n_q_heads / s.n_kv_heads;                          \
    if (s.dtype == kF32) {                                              \
      switch (G_) {                                                     \
        case 1: FN<kF32, 1>(__VA_ARGS__); break;                        \
        case 2: FN<kF32, 2>(__VA_ARGS__); break;                        \
        case 4: FN<kF32, 4>(__VA_ARGS__); break;                        \
        default: FN<kF32, 8>(__VA_ARGS__); break;                       \
      }                                                                 \
    } else if (s.dtype == kBF16) {                                      \
      switch (G_) {                                                     \
        case 1: FN<kBF16, 1>(__VA_ARGS__); break;                       \
        case 2: FN<kBF16, 2>(__VA_ARGS__); break;                       \
        case 4: FN<kBF16, 4>(__VA_ARGS__); break;                       \
        default: FN<kBF16, 8>(__VA_ARGS__); break;                      \
      }                                                                 \
    } else {                                                            \
      switch (G_) {                                                     \
        case 1: FN<kF16, 1>(__VA_ARGS__); break;                        \
        case 2: FN<kF16, 2>(__VA_ARGS__); break;                        \
        case 4: FN<kF16, 4>(__VA_ARGS__); break;                        \
        default: FN<kF16, 8>(__VA_ARGS__); break;                       \
      }                                                                 \
    }                                                                   \
  } while (0)

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
