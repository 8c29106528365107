// Quest block summaries (PRR reference list, Quest): per (sequence b, KV head g, block n) the elementwise min and
// max of the block's keys, read through the paged block table (PagedAttention, PRR reference list).
//
// One wave per block: each load instruction reads 4 token rows (16 lanes x 16 B per 256-byte row); lanes keep
// running min/max, then fold the 4 rows with permlane swaps. Rows 0 and 1 of the wave write the min and max rows.
// Pure HBM streaming: reads bs * 256 B per block, writes 512 B. A last block that the sequence ends inside is
// summarised over the tokens it holds. With the mean-key scorer the same pass sums the rows in fp32 and row 0 of the
// wave writes the block's mean key in fp32 into the slot.
//
// append_kernel: the decode step's new token (position ctx_len - 1) into the K and V caches and its block's summary
// updated in place (min/max, or the running mean), 16 lanes per (b, g).
#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

template <int DT>
__global__ __launch_bounds__(256) void summaries_kernel(const uint8_t* __restrict__ k_cache,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ ids, int64_t n_jobs,
                                                        int64_t n_total, uint8_t* __restrict__ summ, int Hkv, int N,
                                                        int bs, int page, int pps, int last_len, int scorer) {
  using V = Vec<DT>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t job = (int64_t)blockIdx.x * 4 + wave;
  if (job >= n_jobs) return;
  const int64_t flat = ids ? (int64_t)ids[job] : job;   // (b * Hkv + g) * N + n
  if (flat < 0 || flat >= n_total) return;                 // ids outside the summaries are ignored
  const int n = (int)(flat % N);
  const int64_t bg = flat / N;
  const int g = (int)(bg % Hkv);
  const int b = (int)(bg / Hkv);
  const int row = lane >> 4, col = lane & 15;
  const int32_t* trow = table + (int64_t)b * pps;

  const int tok0 = n * bs;
  const int len = block_len(n, N, bs, last_len);
  uint8_t* slot = summ + flat * 2 * kRowBytes;
  if (scorer == kScorerMean) {   // fp32 mean key: lane col sums dims VE * col .. over its row's tokens, then folds
    float sm[V::n];
#pragma unroll
    for (int e = 0; e < V::n; ++e) sm[e] = 0.f;
    for (int t = 0; t < len; t += 4) {
      if (t + row >= len) break;
      const int tok = tok0 + t + row;
      const int64_t phys = trow[tok / page];
      float x[V::n];
      V::to_f32(ld16(k_cache + ((phys * Hkv + g) * page + (tok % page)) * (int64_t)kRowBytes + col * 16), x);
#pragma unroll
      for (int e = 0; e < V::n; ++e) sm[e] += x[e];
    }
    const float inv = 1.f / (float)len;
#pragma unroll
    for (int e = 0; e < V::n; ++e) sm[e] = sum_xor32(sum_xor16(sm[e])) * inv;
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < V::n; e += 4)
        st16(slot + (col * V::n + e) * 4, make_uint4(__float_as_uint(sm[e]), __float_as_uint(sm[e + 1]),
                                                     __float_as_uint(sm[e + 2]), __float_as_uint(sm[e + 3])));
    } else if (row == 1 && V::n * 16 * 4 < 2 * kRowBytes) {   // fp32 storage: the second half of the slot is unused
      st16(slot + kRowBytes + col * 16, make_uint4(0u, 0u, 0u, 0u));
    }
    return;
  }
  float mn[V::n], mx[V::n];
#pragma unroll
  for (int e = 0; e < V::n; ++e) { mn[e] = __builtin_huge_valf(); mx[e] = -__builtin_huge_valf(); }
#pragma unroll 4
  for (int t = 0; t < len; t += 4) {
    if (t + row >= len) break;   // rows past the sequence's end (only in its last block)
    const int tok = tok0 + t + row;
    const int64_t phys = trow[tok / page];
    const uint8_t* p = k_cache + ((phys * Hkv + g) * page + (tok % page)) * (int64_t)kRowBytes + col * 16;
    float x[V::n];
    V::to_f32(ld16(p), x);
#pragma unroll
    for (int e = 0; e < V::n; ++e) { mn[e] = fminf(mn[e], x[e]); mx[e] = fmaxf(mx[e], x[e]); }
  }
#pragma unroll
  for (int e = 0; e < V::n; ++e) {
    Pair p = swap16(mn[e], mn[e]); mn[e] = fminf(p.a, p.b);
    p = swap32(mn[e], mn[e]);      mn[e] = fminf(p.a, p.b);
    p = swap16(mx[e], mx[e]);      mx[e] = fmaxf(p.a, p.b);
    p = swap32(mx[e], mx[e]);      mx[e] = fmaxf(p.a, p.b);
  }
  if (row < 2) {
    uint8_t* dst = summ + (flat * 2 + row) * (int64_t)kRowBytes + col * 16;
    st16(dst, V::from_f32(row == 0 ? mn : mx));
  }
}

template <int DT>
__global__ __launch_bounds__(256) void append_kernel(const uint8_t* __restrict__ k_new,
                                                     const uint8_t* __restrict__ v_new, uint8_t* __restrict__ k_cache,
                                                     uint8_t* __restrict__ v_cache, const int32_t* __restrict__ table,
                                                     uint8_t* __restrict__ summ, int rows, int Hkv, int N, int bs,
                                                     int page, int pps, int pos, int scorer) {
  using V = Vec<DT>;
  const int r = (int)((blockIdx.x * 256 + threadIdx.x) >> 4);   // (b, g) row
  if (r >= rows) return;
  const int col = threadIdx.x & 15;
  const int b = r / Hkv, g = r % Hkv;
  const int64_t phys = table[(int64_t)b * pps + pos / page];
  const int64_t off = ((phys * Hkv + g) * page + pos % page) * (int64_t)kRowBytes + col * 16;
  const uint4 k = ld16(k_new + (int64_t)r * kRowBytes + col * 16);
  st16(k_cache + off, k);
  st16(v_cache + off, ld16(v_new + (int64_t)r * kRowBytes + col * 16));
  uint8_t* slot = summ + (((int64_t)r * N + pos / bs) * 2) * kRowBytes;
  if (scorer == kScorerMean) {   // running fp32 mean: m' = k when the token opens the block, else m + (k - m) / c
    float x[V::n], m[V::n];
    V::to_f32(k, x);
    uint8_t* dst = slot + col * V::n * 4;
    const int c = pos % bs;   // tokens already in the block
    if (c == 0) {
#pragma unroll
      for (int e = 0; e < V::n; ++e) m[e] = x[e];
      if (V::n * 16 * 4 < 2 * kRowBytes) st16(slot + kRowBytes + col * 16, make_uint4(0u, 0u, 0u, 0u));
    } else {
      const float inv = 1.f / (float)(c + 1);
#pragma unroll
      for (int e = 0; e < V::n; e += 4) {
        const uint4 w = ld16(dst + e * 4);
        m[e] = __uint_as_float(w.x); m[e + 1] = __uint_as_float(w.y);
        m[e + 2] = __uint_as_float(w.z); m[e + 3] = __uint_as_float(w.w);
      }
#pragma unroll
      for (int e = 0; e < V::n; ++e) m[e] = fmaf(x[e] - m[e], inv, m[e]);
    }
#pragma unroll
    for (int e = 0; e < V::n; e += 4)
      st16(dst + e * 4, make_uint4(__float_as_uint(m[e]), __float_as_uint(m[e + 1]), __float_as_uint(m[e + 2]),
                                   __float_as_uint(m[e + 3])));
    return;
  }
  uint8_t* smin = slot + col * 16;
  uint8_t* smax = smin + kRowBytes;
  if (pos % bs == 0) {   // the token opens its block
    st16(smin, k);
    st16(smax, k);
    return;
  }
  float x[V::n], lo[V::n], hi[V::n];
  V::to_f32(k, x);
  V::to_f32(ld16(smin), lo);
  V::to_f32(ld16(smax), hi);
#pragma unroll
  for (int e = 0; e < V::n; ++e) { lo[e] = fminf(lo[e], x[e]); hi[e] = fmaxf(hi[e], x[e]); }
  st16(smin, V::from_f32(lo));
  st16(smax, V::from_f32(hi));
}

prr_status launch_append(const prr_shape& s, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* table, void* summ, hipStream_t stream) {
  const int rows = s.batch * s.n_kv_heads;
  const int pos = (s.ctx_len > 0 ? s.ctx_len : s.n_blocks * s.block_size) - 1;
  const dim3 grid((unsigned)((rows * 16 + 255) / 256)), block(256);
  const auto* kn = static_cast<const uint8_t*>(k_new);
  const auto* vn = static_cast<const uint8_t*>(v_new);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  auto* sm = static_cast<uint8_t*>(summ);
#define PRR_APPEND(DT)                                                                                             \
  append_kernel<DT><<<grid, block, 0, stream>>>(kn, vn, kc, vc, table, sm, rows, s.n_kv_heads, s.n_blocks,           \
                                                s.block_size, s.page_size, s.pages_per_seq, pos, s.scorer)
  switch (s.dtype) {
    case kF32: PRR_APPEND(kF32); break;
    case kBF16: PRR_APPEND(kBF16); break;
    default: PRR_APPEND(kF16); break;
  }
#undef PRR_APPEND
  return check_launch("append_kv");
}

prr_status launch_summaries(const prr_shape& s, const void* k_cache, const int32_t* table, const int32_t* ids,
                            int64_t n_jobs, void* summ, hipStream_t stream) {
  if (n_jobs == 0) return PRR_OK;
  const dim3 grid((unsigned)((n_jobs + 3) / 4)), block(256);
  const auto* kc = static_cast<const uint8_t*>(k_cache);
  auto* sm = static_cast<uint8_t*>(summ);
  const int64_t n_total = (int64_t)s.batch * s.n_kv_heads * s.n_blocks;
  trace_begin(PRR_KERNEL_SUMMARIES, stream);
#define PRR_SUMMARIES(DT)                                                                                          \
  summaries_kernel<DT><<<grid, block, 0, stream>>>(kc, table, ids, n_jobs, n_total, sm, s.n_kv_heads, s.n_blocks,   \
                                                   s.block_size, s.page_size, s.pages_per_seq, last_block_len(s),   \
                                                   s.scorer)
  switch (s.dtype) {
    case kF32: PRR_SUMMARIES(kF32); break;
    case kBF16: PRR_SUMMARIES(kBF16); break;
    default: PRR_SUMMARIES(kF16); break;
  }
#undef PRR_SUMMARIES
  trace_end(PRR_KERNEL_SUMMARIES, stream);
  return check_launch("build_summaries");
}

}  // namespace prr
