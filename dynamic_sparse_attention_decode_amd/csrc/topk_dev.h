// topk_dev.h — exact top-K of one row of N <= 32768 fp32 values by one workgroup, lowest index first
// among equal values, written as ascending indices (PRR abstract: attend only to the top-K blocks; the same routine
// forms the EMA predictor's top-K').
//
// Thread t holds the row's values [t*KPT, (t+1)*KPT) in registers as order-preserving uint32 keys. A
// most-significant-digit radix select finds the K-th largest key: the first digit starts at the highest bit in which
// the row's keys differ, 8-bit digits, LDS histogram, early exit when a whole digit bin is taken. Compaction takes
// every key above the threshold class and the lowest-index keys of the threshold class; one workgroup-wide scan
// gives each thread its output offset, so the output comes out in ascending block order. Optionally updates the EMA
// in the same pass. Forced blocks (attention sinks, a local window) carry the largest key; when fewer than K of them
// are present, the radix select runs over the other keys for the remaining places.
//
// Long rows split: a row cut into segments has its top-K among the union of the segments' top-K sets (a key with
// fewer than K keys ahead of it in the row has fewer than K ahead of it in its segment, under the same order of
// value then index). One workgroup per segment writes its top-K as (key, index) candidates in ascending index order,
// the segments one after another, so the candidate list is in ascending block order; one workgroup per row then
// selects the top-K of the candidates with the same tie rule by position.
#pragma once
#include "prr_device.h"
#include "prr_launch.h"

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
  uint32_t red_k[2][16];
  uint32_t red_u[16];
  uint32_t bc[3];
  int flag;
};

__device__ inline uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, d));
  return x;
}

__device__ inline uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, d));
  return x;
}

// Largest and smallest counted key of the workgroup (integer order, so +0 and -0 stay apart as the keys do).
template <int NT, int NK, typename ValidFn>
__device__ inline void block_key_range(const uint32_t (&key)[NK], ValidFn&& valid, uint32_t& kmax, uint32_t& kmin,
                                       TopkLds& L) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t hi = 0u, lo = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < NK; ++j)
    if (valid(j)) { hi = max(hi, key[j]); lo = min(lo, key[j]); }
  hi = wave_max_u32(hi);
  lo = wave_min_u32(lo);
  if (lane == 0) { L.red_k[0][wave] = hi; L.red_k[1][wave] = lo; }
  __syncthreads();
  hi = L.red_k[0][0];
  lo = L.red_k[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { hi = max(hi, L.red_k[0][w]); lo = min(lo, L.red_k[1][w]); }
  kmax = hi;
  kmin = lo;
}

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

// Emits the selected keys (all keys above the radix class, and the first krem keys of the class in order) in
// ascending order: emit(pos, j) for this thread's key j at output slot pos. Thread t holds keys NK per thread in
// index order. Keys for which taken(j) holds are selected whatever the class (forced blocks).
template <int NT, int NK, typename ValidFn, typename EmitFn, typename TakenFn>
__device__ inline void write_selected(const uint32_t (&key)[NK], ValidFn&& valid, const Radix& R, int K, TopkLds& L,
                                      EmitFn&& emit, TakenFn&& taken) {
  const uint32_t pk = shr(R.prefix, R.shift);
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    if (valid(j)) {
      const uint32_t hk = shr(key[j], R.shift);
      const bool t = taken(j);
      cg += t || hk > pk;
      ce += !t && hk == pk;
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
      bool take = taken(j) || hk > pk;
      if (!taken(j) && hk == pk) take = le++ < R.krem;
      if (take) {
        if (pos < (uint32_t)K) emit(pos, j);   // pos < K always holds; the guard keeps a logic error in bounds
        ++pos;
      }
    }
  }
}

// Top-K of the counted keys, emitted in ascending order (see write_selected).
template <int NT, int NK, typename ValidFn, typename EmitFn>
__device__ inline void select_top(const uint32_t (&key)[NK], ValidFn&& valid, int K, TopkLds& L, EmitFn&& emit) {
  uint32_t kmax, kmin;
  block_key_range<NT>(key, valid, kmax, kmin, L);
  const Radix R = radix_select<NT, NK>(key, valid, kmax, kmin, (uint32_t)K, L);
  write_selected<NT, NK>(key, valid, R, K, L, emit, [](int) { return false; });
}

// Top-K when F < K of the counted keys are forced (taken(j)): the other K - F are chosen by the radix select among
// the unforced keys alone, so the forced keys' extreme value does not widen its digit range.
template <int NT, int NK, typename ValidFn, typename TakenFn, typename EmitFn>
__device__ inline void select_top_forced(const uint32_t (&key)[NK], ValidFn&& valid, TakenFn&& taken, int K, int F,
                                         TopkLds& L, EmitFn&& emit) {
  auto free_key = [&](int j) { return valid(j) && !taken(j); };
  uint32_t kmax, kmin;
  block_key_range<NT>(key, free_key, kmax, kmin, L);
  const Radix R = radix_select<NT, NK>(key, free_key, kmax, kmin, (uint32_t)(K - F), L);
  write_selected<NT, NK>(key, valid, R, K, L, emit, taken);
}

// Forced blocks of a row of n blocks: the first `sink` and the last `local` (attention sinks and the local window,
// StreamingLLM in the PRR reference list) take the largest key, so they rank above every score (an fp32 score's key
// is below 0xFFFFFFFF, which only a NaN would reach) and among themselves by index. base: the row position of the
// values at hand (a segment's offset).
struct Force {
  int base = 0, n = 0, sink = 0, local = 0;
  __device__ bool operator()(int i) const { return base + i < sink || base + i >= n - local; }
  // forced positions among [base, base + len)
  __device__ int count(int len) const {
    const int a = max(0, min(sink, base + len) - base);
    const int b = max(0, base + len - max(n - local, base));
    return a + b;
  }
};

// Top-K of one row of N <= NT * KPT values (optionally after the EMA update e = alpha e + (1 - alpha) v, written
// back), by one workgroup of NT threads (256 <= NT <= 1024): emit(pos, i, key) receives the K selected row
// positions i in ascending order, with their keys.
template <int NT, int KPT, bool EMA, typename EmitFn>
__device__ void topk_row_emit(const float* __restrict__ v, float* __restrict__ e_row, float alpha, int first, int N,
                              int K, EmitFn&& emit, Force force = Force{}, const float* __restrict__ conf_s = nullptr,
                              float conf_c = 0.f) {
  static_assert(NT >= 256 && NT <= 1024 && NT % 64 == 0, "workgroup size");
  __shared__ TopkLds L;
  const int i0 = threadIdx.x * KPT;

  // ---- load (and EMA update) --------------------------------------------------------------------------------
  float x[KPT];
  if (KPT % 4 == 0 && ((uintptr_t)v & 15) == 0 && (!EMA || ((uintptr_t)e_row & 15) == 0) && i0 + KPT <= N) {
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

  if (conf_s) {   // the values are an EMA row: rank its optimistic scores u = e + c |s - e| instead
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const float sv = i0 + k < N ? conf_s[i0 + k] : 0.f;
      x[k] = __fadd_rn(x[k], __fmul_rn(conf_c, fabsf(__fsub_rn(sv, x[k]))));
    }
  }
  uint32_t key[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) key[k] = force(i0 + k) ? 0xFFFFFFFFu : f2key(x[k]);
  auto valid = [&](int k) { return i0 + k < N; };
  auto out = [&](uint32_t pos, int j) { emit(pos, i0 + j, key[j]); };
  const int F = force.count(N);
  if (F > 0 && F < K)
    select_top_forced<NT, KPT>(key, valid, [&](int k) { return force(i0 + k); }, K, F, L, out);
  else   // no forced block, or K of them at most: the forced keys take the first places by index
    select_top<NT, KPT>(key, valid, K, L, out);
}

// Smallest key of the workgroup (0xffffffff when no thread holds one).
template <int NT>
__device__ inline uint32_t block_min_u32(uint32_t x, TopkLds& L) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_min_u32(x);
  if (lane == 0) L.red_k[1][wave] = x;
  __syncthreads();
  uint32_t r = L.red_k[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = min(r, L.red_k[1][w]);
  __syncthreads();
  return r;
}

// The next step's predicted set of one row under a per-row budget (BudgetDev; the host has validated it), by one
// workgroup of NT threads, N <= NT * KPT. With EMA the row's average is updated first (e = s on the first step, else
// alpha e + (1 - alpha) s, written back), otherwise e_row already holds it. The row's size k_r is cap (fixed),
// K + ceil(beta m) clamped to [k_min, cap] (misses: m the row's missed blocks at its last completed step, an fp32
// product), or the number of blocks whose optimistic score u = e + c |s - e| (fp32) reaches the K-th EMA key in the
// selection order, clamped (confidence). orow[0, k_r) receives the top-k_r of the EMA (fixed, misses) or of u
// (confidence), forced blocks first, ascending; orow[k_r, cap) = -1.
template <int NT, int KPT, bool EMA>
__device__ void predict_row(const float* __restrict__ s_row, float* e_row, float alpha, int first, int N, int cap,
                            const BudgetDev& bp, int64_t row, int32_t* __restrict__ orow, Force force) {
  static_assert(NT >= 256 && NT <= 1024 && NT % 64 == 0, "workgroup size");
  __shared__ TopkLds L;
  const int i0 = threadIdx.x * KPT;
  const bool conf = bp.policy == 2;
  // keys of the EMA (key) and, for the confidence rule, of the optimistic score u (ukey); forced blocks the largest
  uint32_t key[KPT], ukey[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = i0 + k;
    float e = 0.f, sv = 0.f;
    if (i < N) {
      if (EMA || conf) sv = s_row[i];
      if (EMA) {
        e = first ? sv : fmaf(alpha, e_row[i], (1.f - alpha) * sv);
        e_row[i] = e;
      } else {
        e = e_row[i];
      }
    }
    const bool f = force(i);
    key[k] = f ? 0xFFFFFFFFu : f2key(e);
    ukey[k] = f ? 0xFFFFFFFFu : f2key(__fadd_rn(e, __fmul_rn(bp.c, fabsf(__fsub_rn(sv, e)))));
  }
  auto valid = [&](int k) { return i0 + k < N; };
  int kr = cap;
  if (bp.policy == 1) {
    const float grow = fminf(ceilf(bp.beta * (float)bp.missed_prev[row]), (float)cap);   // cap bounds k_r anyway
    kr = min(max(bp.top_k + (int)grow, bp.k_min), cap);
  } else if (conf) {
    // theta: the K-th largest EMA key
    uint32_t kmax, kmin;
    block_key_range<NT>(key, valid, kmax, kmin, L);
    const Radix R = radix_select<NT, KPT>(key, valid, kmax, kmin, (uint32_t)bp.top_k, L);
    uint32_t theta = R.prefix;
    if (R.shift > 0) {   // the selection took its last digit class whole: theta is that class's smallest key
      const uint32_t pk = shr(R.prefix, R.shift);
      uint32_t lo = 0xffffffffu;
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if (valid(k) && shr(key[k], R.shift) == pk) lo = min(lo, key[k]);
      theta = block_min_u32<NT>(lo, L);
    }
    uint32_t cnt = 0;   // optimistic scores reaching theta
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      cnt += valid(k) && ukey[k] >= theta;
      key[k] = ukey[k];
    }
    uint32_t total;
    block_scan<NT>(cnt, total, L);
    kr = min(max((int)total, bp.k_min), cap);
  }
  auto out = [&](uint32_t pos, int j) { orow[pos] = i0 + j; };
  const int F = force.count(N);
  if (F > 0 && F < kr)
    select_top_forced<NT, KPT>(key, valid, [&](int k) { return force(i0 + k); }, kr, F, L, out);
  else
    select_top<NT, KPT>(key, valid, kr, L, out);
  for (int j = kr + (int)threadIdx.x; j < cap; j += NT) orow[j] = -1;
}

// Top-K of one row into orow (and lds_out, an LDS copy, when given) as K ascending indices.
template <int NT, int KPT, bool EMA>
__device__ inline void topk_row(const float* __restrict__ v, float* __restrict__ e_row, float alpha, int first, int N,
                                int K, int32_t* __restrict__ orow, int32_t* lds_out, Force force) {
  topk_row_emit<NT, KPT, EMA>(v, e_row, alpha, first, N, K, [&](uint32_t pos, int i, uint32_t) {
    orow[pos] = i;
    if (lds_out) lds_out[pos] = i;
  }, force);
}

// ---- long rows: segments, then a merge ---------------------------------------------------------------------------

// Segment s (seg values from s * seg) of a row of N values: its top-min(K, length) as (key, index) candidates at
// ckey_row / cidx_row + s * min(K, seg), ascending by index.
template <int NT, int KPT, bool EMA>
__device__ inline void topk_segment(const float* __restrict__ v_row, float* __restrict__ e_row, float alpha, int first,
                                    int N, int K, int seg, int s, uint32_t* __restrict__ ckey_row,
                                    int32_t* __restrict__ cidx_row, int sink, int local,
                                    const float* __restrict__ conf_s_row = nullptr, float conf_c = 0.f) {
  const int base = s * seg;
  const int n = min(seg, N - base);
  const int kc = min(K, seg);
  uint32_t* ok = ckey_row + (int64_t)s * kc;
  int32_t* oi = cidx_row + (int64_t)s * kc;
  topk_row_emit<NT, KPT, EMA>(v_row + base, EMA ? e_row + base : nullptr, alpha, first, n, min(K, n),
                              [&](uint32_t pos, int i, uint32_t key) {
                                ok[pos] = key;
                                oi[pos] = base + i;
                              },
                              Force{base, N, sink, local}, conf_s_row ? conf_s_row + base : nullptr, conf_c);
}

// Top-K of a row's C candidates (C <= NT * KPT) into orow (and lds_out) as K ascending block indices.
template <int NT, int KPT>
__device__ void topk_merge_row(const uint32_t* __restrict__ ckey_row, const int32_t* __restrict__ cidx_row, int C,
                               int K, int32_t* __restrict__ orow, int32_t* lds_out = nullptr) {
  __shared__ TopkLds L;
  const int i0 = threadIdx.x * KPT;
  uint32_t key[KPT];
  if (KPT % 4 == 0 && ((uintptr_t)ckey_row & 15) == 0 && i0 + KPT <= C) {
#pragma unroll
    for (int k = 0; k < KPT; k += 4) {
      const uint4 a = *reinterpret_cast<const uint4*>(ckey_row + i0 + k);
      key[k] = a.x; key[k + 1] = a.y; key[k + 2] = a.z; key[k + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) key[k] = i0 + k < C ? ckey_row[i0 + k] : 0u;
  }
  auto valid = [&](int k) { return i0 + k < C; };
  select_top<NT, KPT>(key, valid, K, L, [&](uint32_t pos, int j) {
    const int32_t b = cidx_row[i0 + j];
    orow[pos] = b;
    if (lds_out) lds_out[pos] = b;
  });
}

// The next predicted set of a long row under a budget, from segment candidates (ascending block order): misses:
// the top-k_r of the EMA candidates (ekey/eidx, C_e of them, at least cap per segment); confidence: theta = the K-th
// largest EMA candidate key (the segments' top-K, so the row's K-th is among them), k_r = the optimistic-score
// candidates (ukey/uidx: each segment's top-cap of u) at or above theta, clamped, which equals the count over the
// whole row clamped to cap, then their top-k_r. Writes orow[0, k_r) and -1 up to cap.
template <int NT, int KPT>
__device__ void topk_merge_budget_row(const uint32_t* __restrict__ ekey, const int32_t* __restrict__ eidx, int Ce,
                                      const uint32_t* __restrict__ ukey, const int32_t* __restrict__ uidx, int Cu,
                                      int cap, const BudgetDev& bp, int64_t row, int32_t* __restrict__ orow) {
  __shared__ TopkLds L;
  const int i0 = threadIdx.x * KPT;
  int kr = cap;
  if (bp.policy == 1) {
    const float grow = fminf(ceilf(bp.beta * (float)bp.missed_prev[row]), (float)cap);
    kr = min(max(bp.top_k + (int)grow, bp.k_min), cap);
    topk_merge_row<NT, KPT>(ekey, eidx, Ce, kr, orow);
  } else {
    uint32_t key[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) key[k] = i0 + k < Ce ? ekey[i0 + k] : 0u;
    auto valid_e = [&](int k) { return i0 + k < Ce; };
    uint32_t kmax, kmin;
    block_key_range<NT>(key, valid_e, kmax, kmin, L);
    const Radix R = radix_select<NT, KPT>(key, valid_e, kmax, kmin, (uint32_t)bp.top_k, L);
    uint32_t theta = R.prefix;
    if (R.shift > 0) {
      const uint32_t pk = shr(R.prefix, R.shift);
      uint32_t lo = 0xffffffffu;
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if (valid_e(k) && shr(key[k], R.shift) == pk) lo = min(lo, key[k]);
      theta = block_min_u32<NT>(lo, L);
    }
    auto valid_u = [&](int k) { return i0 + k < Cu; };
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      key[k] = i0 + k < Cu ? ukey[i0 + k] : 0u;
      cnt += valid_u(k) && key[k] >= theta;
    }
    uint32_t total;
    block_scan<NT>(cnt, total, L);
    kr = min(max((int)total, bp.k_min), cap);
    select_top<NT, KPT>(key, valid_u, kr, L, [&](uint32_t pos, int j) { orow[pos] = uidx[i0 + j]; });
  }
  for (int j = kr + (int)threadIdx.x; j < cap; j += NT) orow[j] = -1;
}

// Split of a row of N values into segments of seg for a top-K: S segments, kc candidate slots per segment, C
// candidates in all (the last segment may hold fewer).
struct TopkSplit {
  int S, seg, kc, C;
};

__host__ __device__ inline TopkSplit topk_split(int N, int K, int seg) {
  TopkSplit p;
  p.seg = seg;
  p.S = (N + seg - 1) / seg;
  p.kc = K < seg ? K : seg;
  const int last = N - (p.S - 1) * seg;
  p.C = (p.S - 1) * p.kc + (p.kc < last ? p.kc : last);
  return p;
}

// Values per thread (a power of two) of an nt-thread workgroup for a row of n values.
inline int topk_kpt_nt(int n, int nt) {
  int kpt = 1;
  while (kpt * nt < n) kpt *= 2;
  return kpt;
}

// Values per thread of a 1024-thread workgroup for a row of N values (N <= 32768).
inline int topk_kpt(int n) { return topk_kpt_nt(n, 1024); }

}  // namespace prr
