// attn_wave.h — the block-sparse decode-attention tile routine shared by speculation and repair.
//
// Work unit: one wave processes one (sequence b, KV head g, block) for all G query heads of the group. Each load
// instruction reads 4 token rows of K (16 lanes x 16 B per 256-byte row, lane = 16*row + col) and the same 4 rows
// of V, coalesced, through the paged block table (PagedAttention, PRR reference list). Per token the group's G
// logits are full 16-lane DPP sums; the running max is kept uniform across the wave, while l and the O accumulator
// stay per-lane partial sums over the lane's token rows until the end, when two permlane swaps fold the 4 rows (each
// lane then owns G*VE/4 outputs). Logits are kept in log2 units (q pre-scaled by softmax_scale * log2 e) so every
// exponential is one exp2 (online softmax, FlashAttention-2 in the PRR reference list).
//
// Partial record (per (b, g, slot)): m[G] (log2 units), l[G], zero padding to a multiple of 4 floats, then O[G][D]
// (unnormalised), fp32; records are 16-byte aligned.
#pragma once
#include <type_traits>

#include "attn_mfma.h"
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

  static constexpr bool kPipelined = G <= 4;   // two chunk buffers fit the register budget
  static constexpr int64_t kSpecRecBytes = spec_rec_bytes(kF32, G, 16 * Vec<DT>::n);   // fp32 records

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

  // Loads of one chunk of 16 tokens: rows 4*j + row of K and V (j < 4).
  struct Chunk {
    uint4 kv[4], vv[4];
  };

  // len: tokens the block holds (bs, or fewer in a sequence's last block).
  __device__ void load_chunk(Chunk& c, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                             const int32_t* __restrict__ trow, int n, int t0, int bs, int len, int page, int Hkv,
                             int g) const {
    const int64_t tok0 = (int64_t)n * bs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tok = tok0 + t0 + 4 * j + row;
      if (t0 + 4 * j + row < len) {
        const int64_t phys = trow[tok / page];
        const int64_t off = ((phys * Hkv + g) * page + tok % page) * (int64_t)kRowBytes + col * 16;
        c.kv[j] = ld16_stream(kc + off);
        c.vv[j] = ld16_stream(vc + off);
      } else {
        c.kv[j] = make_uint4(0, 0, 0, 0);
        c.vv[j] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Loads of one chunk whose 16 token rows are contiguous from base_k / base_v (nvalid of them exist).
  __device__ void load_chunk_at(Chunk& c, const uint8_t* __restrict__ base_k, const uint8_t* __restrict__ base_v,
                                int nvalid) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = (4 * j + row) * kRowBytes + col * 16;
      c.kv[j] = 4 * j + row < nvalid ? ld16_stream(base_k + off) : make_uint4(0, 0, 0, 0);
      c.vv[j] = 4 * j + row < nvalid ? ld16_stream(base_v + off) : make_uint4(0, 0, 0, 0);
    }
  }

  // Fold one loaded chunk (tokens t0 .. t0 + 15 of a block holding len tokens) into the running state.
  __device__ void compute_chunk(const Chunk& c, int t0, int len) {
    float z[4][G];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = t0 + 4 * j + row < len;
      float x[VE];
      V::to_f32(c.kv[j], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) s = fmaf(q[h][e], x[e], s);
        s = row_sum16(s);
        z[j][h] = ok ? s : -__builtin_huge_valf();
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
      V::to_f32(c.vv[j], y);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] = fmaf(z[j][h], y[e], acc[h][e]);
      }
    }
  }

  // Fold block n (bs tokens apart, holding len of them) into the running state.
  __device__ void block(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                        const int32_t* __restrict__ trow, int n, int bs, int len, int page, int Hkv, int g) {
    for (int t0 = 0; t0 < len; t0 += 16) {
      Chunk c;
      load_chunk(c, kc, vc, trow, n, t0, bs, len, page, Hkv, g);
      compute_chunk(c, t0, len);
    }
  }

  // A stored record's values as one lane needs them: m[G], l[G] and the O slices of the heads this lane's row adds
  // (heads h with h % 4 == row), VE dims at VE*col.
  struct Rec {
    float m[G], l[G];
    float4 o[(G + 3) / 4][VE / 4];
  };

  __device__ void load_record(Rec& r, const float* __restrict__ rec) const {
#pragma unroll
    for (int h = 0; h < G; ++h) { r.m[h] = rec[h]; r.l[h] = rec[G + h]; }
#pragma unroll
    for (int k = 0; k < (G + 3) / 4; ++k) {
      const int h = row + 4 * k;
#pragma unroll
      for (int v = 0; v < VE / 4; ++v)
        r.o[k][v] = h < G ? *reinterpret_cast<const float4*>(rec + ML + h * D + col * VE + 4 * v)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  // Merge a loaded record into the running state. The record's l and O are added by one row only (row h % 4), since
  // the rows are summed when the state is folded.
  __device__ void apply_record(const Rec& r) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], r.m[h]);
      const float c_old = exp2f(m[h] - mn);
      const float c_new = exp2f(r.m[h] - mn);
      m[h] = mn;
      const bool mine = row == (h & 3);
      l[h] = l[h] * c_old + (mine ? r.l[h] * c_new : 0.f);
      float o[VE];
#pragma unroll
      for (int v = 0; v < VE / 4; ++v) {
        const float4 t4 = r.o[h >> 2][v];
        o[4 * v] = t4.x; o[4 * v + 1] = t4.y; o[4 * v + 2] = t4.z; o[4 * v + 3] = t4.w;
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[h][e] = acc[h][e] * c_old + (mine ? o[e] * c_new : 0.f);
    }
  }

  // Merge a stored partial record (m[G] log2, l[G], O[G][D]) into the running state.
  __device__ void merge_record(const float* __restrict__ rec) {
    Rec r;
    load_record(r, rec);
    apply_record(r);
  }

  // Speculation records of fp32 storage are fp32 records.
  __device__ void merge_spec_record(const uint8_t* __restrict__ rec) {
    merge_record(reinterpret_cast<const float*>(rec));
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

  // m[h], l[h] of the folded state into dst[0..G), dst[G..2G).
  __device__ void store_ml(float* dst) const {
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) { dst[h] = m[h]; dst[G + h] = l[h]; }
    }
  }

  __device__ void write_spec_record(uint8_t* __restrict__ rec, const float* folded) {
    write_record(reinterpret_cast<float*>(rec), folded);
  }

  // Write the folded state as a record.
  __device__ void write_record(float* __restrict__ rec, const float* folded) {
    store_ml(rec);
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

// The tile used for a storage dtype: matrix-core logits for 16-bit K/V, all-VALU for fp32.
template <int DT, int G>
using Tile = std::conditional_t<DT == kF32, AttnWave<DT, G>, AttnWaveM<(DT == kF32 ? kBF16 : DT), G>>;

// Attention of one wave over `cnt` blocks (ids from id_of(i)), chunk by chunk, with the next chunk's loads issued
// before the current chunk's arithmetic so that two chunks of K/V are in flight. done(i) runs after block i's last
// chunk (for example to write block i's record and reset the state). When every chunk of 16 tokens lies in one page
// (P16: page size a multiple of 16, at most 64 chunks per call), lane k first resolves chunk k's block id and page;
// the chunk loads then need no dependent address load, which would otherwise stall on the loads in flight.
template <bool P16, typename W, typename IdFn, typename DoneFn>
__device__ inline void run_blocks(W& st, int cnt, IdFn&& id_of, DoneFn&& done, const uint8_t* __restrict__ kc,
                                  const uint8_t* __restrict__ vc, const int32_t* __restrict__ trow, int bs,
                                  int page, int Hkv, int g, int N, int last_len) {
  const int cpb = (bs + 15) >> 4;   // chunks per block
  const int total = cnt * cpb;
  if (total <= 0) return;
  if constexpr (!P16) {   // general path (pages smaller than 16 tokens, or large blocks): one chunk at a time
    for (int i = 0; i < cnt; ++i) {
      const int n = id_of(i);
      st.block(kc, vc, trow, n, bs, block_len(n, N, bs, last_len), page, Hkv, g);
      done(i);
    }
    return;
  }
  // P16: the page size is a multiple of 16 and the caller keeps cnt * chunks per block <= 64; lane k also keeps the
  // number of tokens chunk k holds (16, fewer at the end of a block, none past the end of a sequence)
  const int lane = threadIdx.x & 63;
  int my_phys = 0, my_off = 0, my_nv = 0;
  if (lane < total) {
    const int i = lane / cpb;
    const int n = id_of(i);
    const int part = (lane - i * cpb) << 4;
    const int64_t tc = (int64_t)n * bs + part;
    my_phys = trow[tc / page];
    my_off = (int)(tc % page);
    my_nv = block_len(n, N, bs, last_len) - part;
  }
  // two register buffers used alternately (no copies, so the loads of one stay in flight while the other is used)
  typename W::Chunk ca, cb;
  auto load = [&](typename W::Chunk& c, int k) {
    const int phys = __builtin_amdgcn_readlane(my_phys, k);
    const int off = __builtin_amdgcn_readlane(my_off, k);
    const int64_t r = ((int64_t)phys * Hkv + g) * page + off;
    st.load_chunk_at(c, kc + r * kRowBytes, vc + r * kRowBytes, __builtin_amdgcn_readlane(my_nv, k));
  };
  auto compute = [&](const typename W::Chunk& c, int k) {
    const int i = k / cpb, t0 = (k - i * cpb) << 4;
    st.compute_chunk(c, 0, __builtin_amdgcn_readlane(my_nv, k));
    if (t0 + 16 >= bs) done(i);
  };
  if constexpr (W::kPipelined) {
    load(ca, 0);
    for (int k = 0; k < total; k += 2) {
      if (k + 1 < total) load(cb, k + 1);
      compute(ca, k);
      if (k + 1 < total) {
        if (k + 2 < total) load(ca, k + 2);
        compute(cb, k + 1);
      }
    }
  } else {   // tiles too large for two register buffers: one chunk at a time
    for (int k = 0; k < total; ++k) {
      load(ca, k);
      compute(ca, k);
    }
  }
}

// Speculation of the predicted slots [j0, j1) of row `rowid` by one wave: one partial record per slot. Slots from
// the first empty one (a negative id: a budgeted set's padding, which follows every id of its row) are skipped.
template <int DT, int G, bool P16>
__device__ inline void speculate_slots(int64_t rowid, int j0, int j1, int lane, const uint8_t* __restrict__ q,
                                       const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                       const int32_t* __restrict__ table, const int32_t* __restrict__ pred,
                                       int k_spec, float* __restrict__ partials, int Hq, int Hkv, int N, int bs,
                                       int page, int pps, float qscale, int last_len) {
  using W = Tile<DT, G>;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int32_t* prow = pred + rowid * k_spec;
  for (int c = j0; c < j1; c += 64) {   // the wave's slots end at the first empty one
    const unsigned long long empty = __ballot(c + lane < j1 && prow[c + lane] < 0);
    if (empty) {
      j1 = c + __ffsll(empty) - 1;
      break;
    }
  }
  if (j1 <= j0) return;
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  run_blocks<P16>(
      st, j1 - j0,
      [&](int i) { return min(max(prow[j0 + i], 0), N - 1); },   // ids beyond the row are clamped, never a fault
      [&](int i) {
        float folded[W::NK];
        st.fold(folded);
        st.write_spec_record(reinterpret_cast<uint8_t*>(partials) + (rowid * k_spec + j0 + i) * W::kSpecRecBytes,
                             folded);
        st.init(lane);
      },
      kc, vc, table + (int64_t)b * pps, bs, page, Hkv, g, N, last_len);
}

// Speculation of one predicted slot s = (b * Hkv + g) * k_spec + j by one wave: the block's partial record.
template <int DT, int G>
__device__ inline void speculate_slot(int64_t s, int lane, const uint8_t* __restrict__ q,
                                      const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                      const int32_t* __restrict__ table, const int32_t* __restrict__ pred, int k_spec,
                                      float* __restrict__ partials, int Hq, int Hkv, int N, int bs, int page, int pps,
                                      float qscale, int last_len) {
  using W = Tile<DT, G>;
  const int64_t rowid = s / k_spec;
  const int b = (int)(rowid / Hkv), g = (int)(rowid % Hkv);
  const int32_t id = pred[s];
  if (id < 0) return;              // an empty slot (a budgeted set's padding)
  const int n = min(id, N - 1);    // ids beyond the row are clamped: wrong output, never a fault
  W st;
  st.init(lane);
  st.load_q(q + ((int64_t)b * Hq + (int64_t)g * G) * kRowBytes, qscale);
  st.block(kc, vc, table + (int64_t)b * pps, n, bs, block_len(n, N, bs, last_len), page, Hkv, g);
  float folded[W::NK];
  st.fold(folded);
  st.write_spec_record(reinterpret_cast<uint8_t*>(partials) + s * W::kSpecRecBytes, folded);
}

}  // namespace prr
