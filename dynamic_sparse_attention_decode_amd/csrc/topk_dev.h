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

// ---- workgroup helpers ------------------------------------------------------------------------------------------

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

// Shared LDS of the top-K routine (one per workgroup).
struct TopkLds {
  uint32_t hist[256];
  float red_f[2][16];
  uint32_t red_u[16];
  uint32_t bc[3];
  int flag;
};

// Radix state: the K-th largest counted key lies in {x : x >> shift == prefix >> shift}; keys above that class are
// all taken, and krem keys of the class (the lowest-index ones).
struct Radix {
  uint32_t prefix;
  int shift;
  uint32_t krem;
};

// MSD radix select over keys held NK per thread (valid(j) tells whether key[j] is counted): 8-bit digits from the
// highest bit in which kmax and kmin differ, LDS histogram, early exit when a whole digit bin is taken.
template <int NT, int NK, typename ValidFn>
__device__ inline Radix radix_select(const uint32_t (&key)[NK], ValidFn&& valid, uint32_t kmax, uint32_t kmin,
                                     uint32_t k, TopkLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Radix R{kmax, 0, k};
  if (kmax != kmin) {
    R.shift = 32 - __clz(kmax ^ kmin);
    R.prefix = R.shift >= 32 ? 0u : (kmax >> R.shift) << R.shift;
  }
  while (R.shift > 0) {
    const int db = R.shift < 8 ? R.shift : 8;
    const int ns = R.shift - db;
    if (tid < 256) L.hist[tid] = 0u;
    __syncthreads();
    const uint32_t pk = shr(R.prefix, R.shift);
    const uint32_t dmask = (1u << db) - 1u;
#pragma unroll
    for (int j = 0; j < NK; ++j)
      if (valid(j) && shr(key[j], R.shift) == pk) atomicAdd(&L.hist[(key[j] >> ns) & dmask], 1u);
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = L.hist[4 * lane + j];
      const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
      uint32_t above = wave_suffix_incl(lsum, lane) - lsum;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < R.krem && R.krem <= above + c[j]) { L.bc[0] = 4 * lane + j; L.bc[1] = above; L.bc[2] = c[j]; }
        above += c[j];
      }
    }
    __syncthreads();
    const uint32_t bin = L.bc[0];
    R.krem -= L.bc[1];
    R.prefix |= bin << ns;
    R.shift = ns;
    if (L.bc[2] == R.krem) break;   // the whole bin is selected: no further digits needed
  }
  return R;
}

// Exclusive workgroup scan of x; total receives the sum.
template <int NT>
__device__ inline uint32_t block_scan(uint32_t x, uint32_t& total, TopkLds& L) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(x, lane);
  if (lane == 63) L.red_u[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = L.red_u[w];
    before += w < wave ? c : 0u;
    tot += c;
  }
  total = tot;
  __syncthreads();
  return before + incl - x;
}

// Writes the selected indices (all keys above the radix class, and the first krem keys of the class in order)
// in ascending order. Thread t holds keys NK per thread in index order; idx_of(j) gives key j's index.
template <int NT, int NK, typename ValidFn, typename IdxFn>
__device__ inline void write_selected(const uint32_t (&key)[NK], ValidFn&& valid, const Radix& R, int K,
                                      int32_t* __restrict__ orow, int32_t* lds_out, TopkLds& L, IdxFn&& idx_of) {
  const uint32_t pk = shr(R.prefix, R.shift);
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    if (valid(j)) {
      const uint32_t hk = shr(key[j], R.shift);
      cg += hk > pk;
      ce += hk == pk;
    }
  }
  const uint32_t packed = (cg << 16) | ce;   // both totals stay below 65536
  uint32_t total;
  const uint32_t excl = block_scan<NT>(packed, total, L);
  const uint32_t pre_g = excl >> 16, pre_e = excl & 0xffffu;
  uint32_t pos = pre_g + (pre_e < R.krem ? pre_e : R.krem);
  uint32_t le = pre_e;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    if (valid(j)) {
      const uint32_t hk = shr(key[j], R.shift);
      bool take = hk > pk;
      if (hk == pk) take = le++ < R.krem;
      if (take) {
        if (pos < (uint32_t)K) {   // pos < K always holds; the guard keeps a logic error in bounds
          const int32_t i = idx_of(j);
          orow[pos] = i;
          if (lds_out) lds_out[pos] = i;
        }
        ++pos;
      }
    }
  }
}

// Top-K of one row of N <= NT * KPT values (optionally after the EMA update e = alpha e + (1 - alpha) v, written
// back), by one workgroup of NT threads (256 <= NT <= 1024); orow (and lds_out, an LDS copy, when given) receives K
// ascending indices.
template <int NT, int KPT, bool EMA>
__device__ void topk_row(const float* __restrict__ v, float* __restrict__ e_row, float alpha, int first, int N, int K,
                         int32_t* __restrict__ orow, int32_t* lds_out = nullptr) {
  static_assert(NT >= 256 && NT <= 1024 && NT % 64 == 0, "workgroup size");
  constexpr int NW = NT / 64;
  __shared__ TopkLds L;
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

  // ---- keys and the row range ---------------------------------------------------------------------------------
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
  if (lane == 0) { L.red_f[0][wave] = lmax; L.red_f[1][wave] = lmin; }
  __syncthreads();
  float gmax = L.red_f[0][0], gmin = L.red_f[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { gmax = fmaxf(gmax, L.red_f[0][w]); gmin = fminf(gmin, L.red_f[1][w]); }
  const uint32_t kmax = f2key(gmax), kmin = f2key(gmin);

  auto valid = [&](int k) { return i0 + k < N; };
  const Radix R = radix_select<NT, KPT>(key, valid, kmax, kmin, (uint32_t)K, L);
  write_selected<NT, KPT>(key, valid, R, K, orow, lds_out, L, [&](int k) { return i0 + k; });
}

// Values per thread of a 1024-thread workgroup for a row of N values (N <= 32768).
inline int topk_kpt(int n) {
  int kpt = 1;
  while (kpt * 1024 < n) kpt *= 2;
  return kpt;
}

}  // namespace prr
