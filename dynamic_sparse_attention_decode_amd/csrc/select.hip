// Query-aware block scoring and exact top-K selection (PRR abstract: attend only to the top-K KV blocks of each
// query; PRR reference list, Quest: block scores from per-block key min/max), and the EMA predictor's update and
// top-K' (PRR abstract: "lightweight EMA-based predictor").
//
// score_kernel: s[b,g,n] = sum_d Qpos_d * kmax[n,d] + Qneg_d * kmin[n,d] with Qpos_d = sum_h max(q_hd, 0) and
//   Qneg_d = sum_h min(q_hd, 0) over the group's query heads. Because kmin <= kmax, max(q*kmin, q*kmax) equals
//   max(q,0)*kmax + min(q,0)*kmin exactly, so this is Quest's group-summed score as a streaming GEMV: one pass over
//   the summaries (2*D elements per block), HBM-bound. Each wave load covers two blocks (32 lanes per [min;max]
//   pair); the block's dot product is folded with DPP inside 16-lane rows and one permlane16 swap.
//
// topk_kernel: one 1024-thread workgroup per (b, g) row holds the row's N values in registers as order-preserving
//   uint32 keys (thread t owns indices [t*KPT, (t+1)*KPT)). A most-significant-digit radix select finds the K-th
//   largest key: the first digit starts at the highest bit in which the row's keys differ, 8-bit digits, LDS
//   histogram, early exit when a whole digit bin is taken. Compaction takes every key above the threshold class and
//   the lowest-index keys of the threshold class; one workgroup-wide scan gives each thread its output offset, so
//   the output comes out in ascending block order. Optionally updates the EMA in the same pass.
#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

template <int DT, int G>
__global__ __launch_bounds__(256) void score_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ summ,
                                                    float* __restrict__ scores, int Hq, int Hkv, int N, int chunk) {
  using V = Vec<DT>;
  constexpr int U = 8;   // wave loads in flight per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int col = lane & 15, half = (lane >> 4) & 1, pair = lane >> 5;

  float coef[V::n];
#pragma unroll
  for (int e = 0; e < V::n; ++e) coef[e] = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[V::n];
    V::to_f32(ld16(q + ((int64_t)b * Hq + g * G + h) * kRowBytes + col * 16), x);
#pragma unroll
    for (int e = 0; e < V::n; ++e) coef[e] += half ? fmaxf(x[e], 0.f) : fminf(x[e], 0.f);
  }

  const int c0 = blockIdx.x * chunk;
  const int c1 = min(N, c0 + chunk);
  const uint8_t* base = summ + (int64_t)bg * N * (2 * kRowBytes) + half * kRowBytes + col * 16;
  float* srow = scores + (int64_t)bg * N;
  for (int n0 = c0 + wave * 2 + pair; n0 < c1; n0 += 8 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + 8 * u;
      v[u] = n < c1 ? ld16(base + (int64_t)n * (2 * kRowBytes)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[V::n];
      V::to_f32(v[u], x);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < V::n; ++e) s = fmaf(coef[e], x[e], s);
      s = sum_xor16(row_sum16(s));
      const int n = n0 + 8 * u;
      if ((lane & 31) == 0 && n < c1) srow[n] = s;
    }
  }
}

// ---- workgroup helpers for the 1024-thread top-K kernel ----------------------------------------------------------

__device__ inline uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(x, d);
    if (lane >= d) x += t;
  }
  return x;
}

__device__ inline uint32_t wave_suffix_incl(uint32_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_down(x, d);
    if (lane + d < 64) x += t;
  }
  return x;
}

__device__ inline uint32_t shr(uint32_t x, int s) { return s >= 32 ? 0u : x >> s; }

template <int KPT, bool EMA>
__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ vals, float* __restrict__ ema,
                                                    float alpha, int first, int N, int K,
                                                    int32_t* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ float red_f[2][16];
  __shared__ uint32_t red_u[16];
  __shared__ uint32_t bc[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* v = vals + row * N;
  float* e_row = EMA ? ema + row * N : nullptr;
  const int i0 = tid * KPT;

  // ---- load (and EMA update) --------------------------------------------------------------------------------
  float x[KPT];
  if (KPT % 4 == 0 && (N & 3) == 0 && i0 + KPT <= N) {
#pragma unroll
    for (int k = 0; k < KPT; k += 4) {
      const float4 a = *reinterpret_cast<const float4*>(v + i0 + k);
      x[k] = a.x; x[k + 1] = a.y; x[k + 2] = a.z; x[k + 3] = a.w;
    }
    if (EMA) {
#pragma unroll
      for (int k = 0; k < KPT; k += 4) {
        float4 o = *reinterpret_cast<const float4*>(e_row + i0 + k);
        if (!first) {
          o.x = fmaf(alpha, o.x, (1.f - alpha) * x[k]);
          o.y = fmaf(alpha, o.y, (1.f - alpha) * x[k + 1]);
          o.z = fmaf(alpha, o.z, (1.f - alpha) * x[k + 2]);
          o.w = fmaf(alpha, o.w, (1.f - alpha) * x[k + 3]);
        } else {
          o = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
        }
        *reinterpret_cast<float4*>(e_row + i0 + k) = o;
        x[k] = o.x; x[k + 1] = o.y; x[k + 2] = o.z; x[k + 3] = o.w;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int i = i0 + k;
      if (i < N) {
        float s = v[i];
        if (EMA) {
          s = first ? s : fmaf(alpha, e_row[i], (1.f - alpha) * s);
          e_row[i] = s;
        }
        x[k] = s;
      } else {
        x[k] = 0.f;
      }
    }
  }

  // ---- row range of the keys --------------------------------------------------------------------------------
  float lmax = -__builtin_huge_valf(), lmin = __builtin_huge_valf();
  uint32_t key[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool ok = i0 + k < N;
    key[k] = ok ? f2key(x[k]) : 0u;
    if (ok) { lmax = fmaxf(lmax, x[k]); lmin = fminf(lmin, x[k]); }
  }
  lmax = wave_max(lmax);
  lmin = -wave_max(-lmin);
  if (lane == 0) { red_f[0][wave] = lmax; red_f[1][wave] = lmin; }
  __syncthreads();
  float gmax = red_f[0][0], gmin = red_f[1][0];
#pragma unroll
  for (int w = 1; w < 16; ++w) { gmax = fmaxf(gmax, red_f[0][w]); gmin = fminf(gmin, red_f[1][w]); }
  const uint32_t kmax = f2key(gmax), kmin = f2key(gmin);

  // ---- MSD radix select ---------------------------------------------------------------------------------------
  uint32_t prefix = kmax;
  int shift = 0;
  uint32_t krem = (uint32_t)K;
  if (kmax != kmin) {
    const int hb = 31 - __clz(kmax ^ kmin);
    shift = hb + 1;
    prefix = shift >= 32 ? 0u : (kmax >> shift) << shift;
  }
  while (shift > 0) {
    const int db = shift < 8 ? shift : 8;
    const int ns = shift - db;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t pk = shr(prefix, shift);
    const uint32_t dmask = (1u << db) - 1u;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      if (i0 + k < N && shr(key[k], shift) == pk) atomicAdd(&hist[(key[k] >> ns) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[4 * lane + j];
      const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
      uint32_t above = wave_suffix_incl(lsum, lane) - lsum;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < krem && krem <= above + c[j]) { bc[0] = 4 * lane + j; bc[1] = above; bc[2] = c[j]; }
        above += c[j];
      }
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    krem -= bc[1];
    prefix |= bin << ns;
    shift = ns;
    if (bc[2] == krem) break;   // the whole bin is selected: no further digits needed
  }

  // ---- compaction in ascending index order ---------------------------------------------------------------------
  const uint32_t pk = shr(prefix, shift);
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    if (i0 + k < N) {
      const uint32_t hk = shr(key[k], shift);
      cg += hk > pk;
      ce += hk == pk;
    }
  }
  const uint32_t packed = (cg << 16) | ce;
  const uint32_t incl = wave_incl_scan(packed, lane);
  if (lane == 63) red_u[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += red_u[w];
  const uint32_t excl = before + incl - packed;
  const uint32_t pre_g = excl >> 16, pre_e = excl & 0xffffu;
  uint32_t pos = pre_g + (pre_e < krem ? pre_e : krem);
  uint32_t le = pre_e;
  int32_t* orow = out + row * K;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = i0 + k;
    if (i < N) {
      const uint32_t hk = shr(key[k], shift);
      if (hk > pk) {
        if (pos < (uint32_t)K) orow[pos] = i;   // pos < K always holds; the guard keeps a logic error in bounds
        ++pos;
      } else if (hk == pk) {
        if (le < krem) {
          if (pos < (uint32_t)K) orow[pos] = i;
          ++pos;
        }
        ++le;
      }
    }
  }
}

// ---- launchers -----------------------------------------------------------------------------------------------------

template <int DT>
static void score_dispatch(const prr_shape& s, dim3 grid, const uint8_t* q, const uint8_t* sm, float* scores,
                           int chunk, hipStream_t st) {
  const int G = s.n_q_heads / s.n_kv_heads;
  const dim3 blk(256);
  switch (G) {
    case 1: score_kernel<DT, 1><<<grid, blk, 0, st>>>(q, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk); break;
    case 2: score_kernel<DT, 2><<<grid, blk, 0, st>>>(q, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk); break;
    case 4: score_kernel<DT, 4><<<grid, blk, 0, st>>>(q, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk); break;
    default: score_kernel<DT, 8><<<grid, blk, 0, st>>>(q, sm, scores, s.n_q_heads, s.n_kv_heads, s.n_blocks, chunk); break;
  }
}

prr_status launch_score(const prr_shape& s, const void* q, const void* summ, float* scores, hipStream_t stream) {
  const int rows = s.batch * s.n_kv_heads;
  // Blocks per workgroup: a multiple of 64 (one unrolled wave round), sized for about 2048 workgroups in total.
  const int64_t total = (int64_t)rows * s.n_blocks;
  int chunk = (int)((total / 2048 + 63) / 64 * 64);
  if (chunk < 64) chunk = 64;
  const dim3 grid((unsigned)((s.n_blocks + chunk - 1) / chunk), (unsigned)rows);
  const auto* qq = static_cast<const uint8_t*>(q);
  const auto* sm = static_cast<const uint8_t*>(summ);
  trace_begin(PRR_KERNEL_SCORE, stream);
  switch (s.dtype) {
    case kF32: score_dispatch<kF32>(s, grid, qq, sm, scores, chunk, stream); break;
    case kBF16: score_dispatch<kBF16>(s, grid, qq, sm, scores, chunk, stream); break;
    default: score_dispatch<kF16>(s, grid, qq, sm, scores, chunk, stream); break;
  }
  trace_end(PRR_KERNEL_SCORE, stream);
  return check_launch("score");
}

template <bool EMA>
static void topk_dispatch(int kpt, dim3 grid, const float* vals, float* ema, float alpha, int first, int N, int K,
                          int32_t* out, hipStream_t st) {
  const dim3 blk(1024);
  switch (kpt) {
    case 1: topk_kernel<1, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 2: topk_kernel<2, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 4: topk_kernel<4, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 8: topk_kernel<8, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    case 16: topk_kernel<16, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
    default: topk_kernel<32, EMA><<<grid, blk, 0, st>>>(vals, ema, alpha, first, N, K, out); break;
  }
}

prr_status launch_topk(const prr_shape& s, const float* values, float* ema, float alpha, int first, int k,
                       int32_t* out_idx, hipStream_t stream) {
  int kpt = 1;
  while (kpt * 1024 < s.n_blocks) kpt *= 2;
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
