// score_dev.h — Quest block scoring as a streaming GEMV (PRR reference list, Quest), or mean-key scoring, optionally
// fused with the EMA predictor's update (PRR abstract: a light predictor built on an exponential moving average).
//
// s[b,g,n] = sum_d Qpos_d * kmax[n,d] + Qneg_d * kmin[n,d] with Qpos_d = sum_h max(q_hd, 0) and
// Qneg_d = sum_h min(q_hd, 0) over the group's query heads. Because kmin <= kmax, max(q*kmin, q*kmax) equals
// max(q,0)*kmax + min(q,0)*kmin exactly, so this is Quest's group-summed score read in one pass over the summaries
// (2*D elements per block), HBM-bound. Each wave load covers two blocks (32 lanes per [min;max] pair); the block's
// dot product is folded with DPP inside 16-lane rows and one permlane16 swap.
#pragma once
#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

// Scores of blocks [bx * chunk, (bx + 1) * chunk) of row bg = b * Hkv + g, by one 256-thread workgroup. With EMA
// the same pass updates the row's average in place: e = s on the first step, else alpha e + (1 - alpha) s.
template <int DT, int G, bool EMA>
__device__ inline void score_chunk(int bx, int bg, const uint8_t* __restrict__ q, const uint8_t* __restrict__ summ,
                                   float* __restrict__ scores, int Hq, int Hkv, int N, int chunk,
                                   float* __restrict__ ema, float alpha, int first) {
  using V = Vec<DT>;
  constexpr int U = 8;   // wave loads in flight per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = bg / Hkv, g = bg % Hkv;
  const int col = lane & 15, half = (lane >> 4) & 1, pair = lane >> 5;

  // the query rows and the first round of summary loads are issued together (one memory round trip, not two)
  uint4 qraw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qraw[h] = ld16(q + ((int64_t)b * Hq + g * G + h) * kRowBytes + col * 16);

  const int c0 = bx * chunk;
  const int c1 = min(N, c0 + chunk);
  const uint8_t* base = summ + (int64_t)bg * N * (2 * kRowBytes) + half * kRowBytes + col * 16;
  float* srow = scores + (int64_t)bg * N;
  float* erow = EMA ? ema + (int64_t)bg * N : nullptr;
  const bool owner = (lane & 31) == 0;   // lanes 0 and 32 hold their block's score after the fold
  uint4 v[U];
  float e_old[U];
  auto issue = [&](int m0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = m0 + 8 * u;
      v[u] = n < c1 ? ld16_stream(base + (int64_t)n * (2 * kRowBytes)) : make_uint4(0, 0, 0, 0);
      e_old[u] = (EMA && !first && owner && n < c1) ? erow[n] : 0.f;
    }
  };
  int n0 = c0 + wave * 2 + pair;
  issue(n0);

  float coef[V::n];
#pragma unroll
  for (int e = 0; e < V::n; ++e) coef[e] = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[V::n];
    V::to_f32(qraw[h], x);
#pragma unroll
    for (int e = 0; e < V::n; ++e) coef[e] += half ? fmaxf(x[e], 0.f) : fminf(x[e], 0.f);
  }

  for (; n0 < c1; n0 += 8 * U) {
    if (n0 > c0 + 7) issue(n0);   // rounds after the first
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[V::n];
      V::to_f32(v[u], x);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < V::n; ++e) s = fmaf(coef[e], x[e], s);
      s = sum_xor16(row_sum16(s));
      const int n = n0 + 8 * u;
      if (owner && n < c1) {
        srow[n] = s;
        if (EMA) erow[n] = first ? s : fmaf(alpha, e_old[u], (1.f - alpha) * s);
      }
    }
  }
}

// Mean-key scores (the second scorer) of blocks [bx * chunk, (bx + 1) * chunk) of row bg: s[n] = <sum_h q_h, mean_n>
// with the block's mean key stored in fp32 in its summary slot (dims 64 * half + 4 * col .. + 3 at byte
// 256 * half + 16 * col; with fp32 storage D = 64 and only the first half is used). Same wave layout, fold and EMA
// update as score_chunk.
template <int DT, int G, bool EMA>
__device__ inline void score_chunk_mean(int bx, int bg, const uint8_t* __restrict__ q,
                                        const uint8_t* __restrict__ summ, float* __restrict__ scores, int Hq, int Hkv,
                                        int N, int chunk, float* __restrict__ ema, float alpha, int first) {
  constexpr int U = 8;   // wave loads in flight per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = bg / Hkv, g = bg % Hkv;
  const int col = lane & 15, half = (lane >> 4) & 1, pair = lane >> 5;
  const bool used = DT != kF32 || half == 0;

  // the query values and the first round of summary loads are issued together, as in score_chunk
  uint4 qraw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint8_t* qh = q + ((int64_t)b * Hq + g * G + h) * kRowBytes;
    if (!used) {
      qraw[h] = make_uint4(0u, 0u, 0u, 0u);
    } else if constexpr (DT == kF32) {
      qraw[h] = ld16(qh + col * 16);
    } else {   // the 4 16-bit values at dims 64 * half + 4 * col
      const uint2 w = *reinterpret_cast<const uint2*>(qh + (64 * half + 4 * col) * 2);
      qraw[h] = make_uint4(w.x, w.y, 0u, 0u);
    }
  }

  const int c0 = bx * chunk;
  const int c1 = min(N, c0 + chunk);
  const uint8_t* base = summ + (int64_t)bg * N * (2 * kRowBytes) + half * kRowBytes + col * 16;
  float* srow = scores + (int64_t)bg * N;
  float* erow = EMA ? ema + (int64_t)bg * N : nullptr;
  const bool owner = (lane & 31) == 0;
  uint4 v[U];
  float e_old[U];
  auto issue = [&](int m0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = m0 + 8 * u;
      v[u] = (used && n < c1) ? ld16_stream(base + (int64_t)n * (2 * kRowBytes)) : make_uint4(0, 0, 0, 0);
      e_old[u] = (EMA && !first && owner && n < c1) ? erow[n] : 0.f;
    }
  };
  int n0 = c0 + wave * 2 + pair;
  issue(n0);

  float coef[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[Vec<DT>::n];
    Vec<DT>::to_f32(qraw[h], x);
#pragma unroll
    for (int e = 0; e < 4; ++e) coef[e] += x[e];
  }

  for (; n0 < c1; n0 += 8 * U) {
    if (n0 > c0 + 7) issue(n0);   // rounds after the first
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = coef[0] * __uint_as_float(v[u].x);
      s = fmaf(coef[1], __uint_as_float(v[u].y), s);
      s = fmaf(coef[2], __uint_as_float(v[u].z), s);
      s = fmaf(coef[3], __uint_as_float(v[u].w), s);
      s = sum_xor16(row_sum16(s));
      const int n = n0 + 8 * u;
      if (owner && n < c1) {
        srow[n] = s;
        if (EMA) erow[n] = first ? s : fmaf(alpha, e_old[u], (1.f - alpha) * s);
      }
    }
  }
}

// The shape's scorer over one chunk of a row.
template <int DT, int G, bool EMA>
__device__ inline void score_any(int scorer, int bx, int bg, const uint8_t* __restrict__ q,
                                 const uint8_t* __restrict__ summ, float* __restrict__ scores, int Hq, int Hkv, int N,
                                 int chunk, float* __restrict__ ema, float alpha, int first) {
  if (scorer == kScorerMean)
    score_chunk_mean<DT, G, EMA>(bx, bg, q, summ, scores, Hq, Hkv, N, chunk, ema, alpha, first);
  else
    score_chunk<DT, G, EMA>(bx, bg, q, summ, scores, Hq, Hkv, N, chunk, ema, alpha, first);
}

// Blocks per scoring workgroup, a multiple of one unrolled wave round (4 waves x 2 blocks x 8 loads in flight = 64).
// Scores alone: one round per workgroup, so each issues its loads once and the dispatcher balances the many short
// workgroups across the chip (paged batch, same-box A/B: 16384 workgroups of 64 blocks 81.4 us, against 86.2 us for
// 2048 resident workgroups of 512 blocks and 85.5 us for 4096 of 256). With the EMA update, which adds a load and a
// store per block, about 2048 workgroups (million-token layer: 128 blocks each, 25.4 us, against 27.3 us at 64).
inline int score_chunk_size(const prr_shape& s, bool ema) {
  if (!ema) return 64;
  const int64_t total = (int64_t)s.batch * s.n_kv_heads * s.n_blocks;
  const int chunk = (int)((total / 2048 + 63) / 64 * 64);
  return chunk < 64 ? 64 : chunk;
}

}  // namespace prr
