// topk_dev.h — exact top-K of one row of N <= 32768 fp32 values by one workgroup, lowest index first
// among equal values, written as ascending indices (PRR abstract: attend only to the top-K blocks; the same routine
// forms the EMA predictor's top-K').
//
// Thread t holds the row's values [t*KPT, (t+1)*KPT) in registers as order-preserving uint32 keys. A
// most-significant-digit radix select finds the K-th largest key: the first digit starts at the highest bit in which
// the row's keys differ, 8-bit digits, LDS histogram, early exit when a whole digit bin is taken. Compaction takes
// every key above the threshold class and the lowest-index keys of the threshold class; one workgroup-wide scan
// gives each thread its output offset, so the output comes out in ascending block order. Optionally updates the EMA
// in the same pass.
#pragma once
#include "prr_device.h"

namespace prr {

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

// Top-K of one row of N <= NT * KPT values (optionally after the EMA update e = alpha e + (1 - alpha) v, written
// back), by one workgroup of NT threads (256 <= NT <= 1024); orow (and lds_out, an LDS copy, when given) receives K
// ascending indices.
template <int NT, int KPT, bool EMA>
__device__ void topk_row(const float* __restrict__ v, float* __restrict__ e_row, float alpha, int first, int N, int K,
                         int32_t* __restrict__ orow, int32_t* lds_out = nullptr) {
  static_assert(NT >= 256 && NT <= 1024 && NT % 64 == 0, "workgroup size");
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[256];
  __shared__ float red_f[2][NW];
  __shared__ uint32_t red_u[NW];
  __shared__ uint32_t bc[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  for (int w = 1; w < NW; ++w) { gmax = fmaxf(gmax, red_f[0][w]); gmin = fminf(gmin, red_f[1][w]); }
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
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = i0 + k;
    if (i < N) {
      const uint32_t hk = shr(key[k], shift);
      if (hk > pk) {
        if (pos < (uint32_t)K) {   // pos < K always holds; the guard keeps a logic error in bounds
          orow[pos] = i;
          if (lds_out) lds_out[pos] = i;
        }
        ++pos;
      } else if (hk == pk) {
        if (le < krem) {
          if (pos < (uint32_t)K) {
            orow[pos] = i;
            if (lds_out) lds_out[pos] = i;
          }
          ++pos;
        }
        ++le;
      }
    }
  }
}

// Values per thread of a 1024-thread workgroup for a row of N values (N <= 32768).
inline int topk_kpt(int n) {
  int kpt = 1;
  while (kpt * 1024 < n) kpt *= 2;
  return kpt;
}

}  // namespace prr
