// attn_mfma.h — block-sparse decode-attention tile for 16-bit K/V on gfx950: logits on the matrix cores, p.V on the
// vector ALUs in fp32.
//
// Per chunk of 16 tokens of one block and the G query heads of one KV head:
//  * S^T = K . Q^T with four v_mfma_f32_16x16x32_{bf16,f16} (k = 128 head dims in 4 slices of 32). The A operand is
//    the K tile as stored (lane l: token l%16, 8 dims at 8*(l/16) + 32*kk), the B operand the group's queries (lane l:
//    head l%16, zero beyond G), loaded once. Products of 16-bit values are exact in fp32, so the logits keep the
//    precision of an fp32 dot product. The result lands with lane l holding tokens 4*(l/16)+r of head l%16.
//  * Online softmax per head in log2 units (m uniform over the wave's rows after two permlane max-swaps).
//  * O += p . V in fp32 on the vector ALUs: lane (row, col) loads V rows 4*row+r, dims 8*col.., and takes p of head
//    h from lane 16*row + h of its row with a ds_swizzle broadcast.
// Compared with an all-VALU tile this removes the K-side conversions, FMAs and DPP reductions (about two thirds of
// the vector instructions per byte), which otherwise bound the tile below the HBM rate.
#pragma once
#include "prr_device.h"
#include "prr_launch.h"

namespace prr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ inline floatx4_t mfma16x16x32(const uint4 a, const uint4 b, floatx4_t c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// value of `x` in lane 16*(lane/16) + h (broadcast within each 16-lane row)
template <int H>
__device__ inline float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (H << 5)));
}

template <int DT, int G>
struct AttnWaveM {
  using V = Vec<DT>;
  static constexpr int VE = V::n;       // 8
  static constexpr int D = 16 * VE;     // 128
  static constexpr int NV = G * VE;
  static constexpr int NK = NV / 4;
  static_assert(DT != kF32, "matrix-core tile is for 16-bit storage");
  static constexpr bool kPipelined = G <= 4;   // two chunk buffers fit the register budget
  static constexpr int64_t kSpecRecBytes = spec_rec_bytes(kBF16, G, D);   // speculation records: O in bf16

  uint4 qb[4];        // B operand: query head l%16 (zero beyond G), dims 8*(l/16) + 32*kk
  float qscale;
  float m_l, l_l;     // running max (log2 units) and partial sum of head l%16 over this lane's tokens
  float acc[G][VE];   // partial O over this lane's row tokens, dims 8*col..
  int lane, row, col;

  __device__ void init(int lane_) {
    lane = lane_;
    row = lane >> 4;
    col = lane & 15;
    m_l = -__builtin_huge_valf();
    l_l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;
  }

  __device__ void load_q(const uint8_t* qg, float qs) {   // qg = q + (b*Hq + g*G) * 256
    qscale = qs;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qb[kk] = col < G ? ld16(qg + col * kRowBytes + 16 * row + 64 * kk) : make_uint4(0, 0, 0, 0);
  }

  // Loads of one chunk of 16 tokens: K as the A operand (token col, 8 dims at 8*row + 32*kk) and V rows 4*row + r.
  struct Chunk {
    uint4 ka[4], vv[4];
  };

  // len: tokens the block holds (bs, or fewer in a sequence's last block).
  // phys >= 0: the physical page of the chunk, already looked up (a block inside one page).
  __device__ void load_chunk(Chunk& c, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                             const int32_t* __restrict__ trow, int n, int t0, int bs, int len, int page, int Hkv,
                             int g, int64_t phys = -1) const {
    const int64_t tok0 = (int64_t)n * bs;
    const bool kok = t0 + col < len;
    if ((page & 15) == 0) {   // the 16 tokens share one page
      const int64_t tc = tok0 + t0;
      if (phys < 0) phys = trow[tc / page];
      const uint8_t* base_k = kc + ((phys * Hkv + g) * page + tc % page) * (int64_t)kRowBytes;
      const uint8_t* base_v = vc + ((phys * Hkv + g) * page + tc % page) * (int64_t)kRowBytes;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        c.ka[kk] = kok ? ld16_stream(base_k + col * kRowBytes + 16 * row + 64 * kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 4 * row + r;
        c.vv[r] = t0 + tt < len ? ld16_stream(base_v + tt * kRowBytes + 16 * col) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int64_t tk = tok0 + t0 + col;
      const int64_t pk = kok ? trow[tk / page] : 0;
      const uint8_t* base_k = kc + ((pk * Hkv + g) * page + tk % page) * (int64_t)kRowBytes;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        c.ka[kk] = kok ? ld16_stream(base_k + 16 * row + 64 * kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 4 * row + r;
        const int64_t tv = tok0 + t0 + tt;
        if (t0 + tt < len) {
          const int64_t pv = trow[tv / page];
          c.vv[r] = ld16_stream(vc + ((pv * Hkv + g) * page + tv % page) * (int64_t)kRowBytes + 16 * col);
        } else {
          c.vv[r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  // Loads of one chunk whose 16 token rows are contiguous from base_k / base_v (nvalid of them exist).
  __device__ void load_chunk_at(Chunk& c, const uint8_t* __restrict__ base_k, const uint8_t* __restrict__ base_v,
                                int nvalid) const {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      c.ka[kk] = col < nvalid ? ld16_stream(base_k + col * kRowBytes + 16 * row + 64 * kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = 4 * row + r;
      c.vv[r] = tt < nvalid ? ld16_stream(base_v + tt * kRowBytes + 16 * col) : make_uint4(0, 0, 0, 0);
    }
  }

  // Fold one loaded chunk (tokens t0 .. t0 + 15 of a block holding len tokens) into the running state.
  __device__ void compute_chunk(const Chunk& c, int t0, int len) {
    // ---- logits on the matrix cores --------------------------------------------------------------------------
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s = mfma16x16x32<DT>(c.ka[kk], qb[kk], s);
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = t0 + 4 * row + r < len ? s[r] * qscale : -__builtin_huge_valf();
    // ---- online softmax for head col --------------------------------------------------------------------------
    float mc = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mc = max_xor32(max_xor16(mc));
    const float mn = fmaxf(m_l, mc);
    const float corr = exp2f(m_l - mn);
    m_l = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2f(z[r] - mn);
    l_l = l_l * corr + ((p[0] + p[1]) + (p[2] + p[3]));
    // ---- O = O * corr + p . V (fp32), one V row at a time ---------------------------------------------------
    rescale<0>(corr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float y[VE];
      V::to_f32(c.vv[r], y);
      accumulate_row<0>(p[r], y);
    }
  }

  // Fold block n (bs tokens apart, holding len of them) into the running state.
  __device__ void block(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                        const int32_t* __restrict__ trow, int n, int bs, int len, int page, int Hkv, int g) {
    // a block of several chunks inside one page takes one page lookup for all of them, not one per chunk (131K
    // batch, 64-token blocks, the selection launch's speculation waves, same-box A/B: step 52.6 -> 49.4 us); a
    // one-chunk block keeps the lookup in the chunk load (32K layer: 20.8 against 21.2 us with it hoisted)
    const int64_t phys =
        bs > 16 && (page & 15) == 0 && page % bs == 0 ? (int64_t)trow[(int64_t)n * bs / page] : -1;
    for (int t0 = 0; t0 < len; t0 += 16) {
      Chunk c;
      load_chunk(c, kc, vc, trow, n, t0, bs, len, page, Hkv, g, phys);
      compute_chunk(c, t0, len);
    }
  }

  // acc[h] *= corr of head h (held by lane h)
  template <int H>
  __device__ inline void rescale(float corr) {
    if constexpr (H < G) {
      const float ch = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), H));
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[H][e] *= ch;
      rescale<H + 1>(corr);
    }
  }

  // acc[h] += p(head h, token row r) * y, p of head h taken from lane 16*row + h
  template <int H>
  __device__ inline void accumulate_row(float pr, const float* y) {
    if constexpr (H < G) {
      const float ph = row_bcast<H>(pr);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[H][e] = fmaf(ph, y[e], acc[H][e]);
      accumulate_row<H + 1>(pr, y);
    }
  }

  // A stored record's values as one lane needs them: m[G], l[G] and the O slices of the heads this lane's row adds
  // (heads h with h % 4 == row), 8 dims at 8*col.
  struct Rec {
    float m[G], l[G];
    float4 o[(G + 3) / 4][VE / 4];
  };

  __device__ void load_record(Rec& r, const float* __restrict__ rec) const {
    constexpr int ML = rec_ml(G);
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

  // Merge a loaded record; its l and O enter through one row only.
  __device__ void apply_record(const Rec& r) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_l), h));
      const float mn = fmaxf(mh, r.m[h]);
      const float c_old = exp2f(mh - mn);
      const float c_new = exp2f(r.m[h] - mn);
      if (col == h) {
        m_l = mn;
        l_l = l_l * c_old + (row == 0 ? r.l[h] * c_new : 0.f);
      }
      const bool mine = row == (h & 3);
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

  // Merge a stored record (m[G] log2, l[G], O[G][D]).
  __device__ void merge_record(const float* __restrict__ rec) {
    Rec r;
    load_record(r, rec);
    apply_record(r);
  }

  // A speculation record (fp16 O / l, m and l in fp32) as one lane needs it: O = (O / l) * l.
  __device__ void load_spec_record(Rec& r, const uint8_t* __restrict__ rec) const {
    const float* ml = reinterpret_cast<const float*>(rec);
    const uint16_t* o = reinterpret_cast<const uint16_t*>(rec + rec_ml(G) * 4);
#pragma unroll
    for (int h = 0; h < G; ++h) { r.m[h] = ml[h]; r.l[h] = ml[G + h]; }
#pragma unroll
    for (int k = 0; k < (G + 3) / 4; ++k) {
      const int h = row + 4 * k;
      const float lh = h < G ? ml[G + h] : 0.f;
#pragma unroll
      for (int v = 0; v < VE / 4; ++v) {
        const float4 t = h < G ? unpack_f16x4(*reinterpret_cast<const uint2*>(o + h * D + col * VE + 4 * v))
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        r.o[k][v] = make_float4(t.x * lh, t.y * lh, t.z * lh, t.w * lh);
      }
    }
  }

  __device__ void merge_spec_record(const uint8_t* __restrict__ rec) {
    Rec r;
    load_spec_record(r, rec);
    apply_record(r);
  }

  // Write the folded state as a speculation record: m and l in fp32, O / l in fp16 (rounded to nearest even; l >= 1,
  // since the block's largest logit contributes 2^0).
  __device__ void write_spec_record(uint8_t* __restrict__ rec, const float* folded) const {
    store_ml(reinterpret_cast<float*>(rec));
    uint16_t* o = reinterpret_cast<uint16_t*>(rec + rec_ml(G) * 4);
    if constexpr (NK % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NK; i += 4) {
        const int f = row * NK + i;
        const int h = f / VE, e = f % VE;
        const float il = 1.f / __shfl(l_l, h);   // lane h (row 0, column h) holds head h's l
        *reinterpret_cast<uint2*>(o + h * D + col * VE + e) =
            make_uint2(pack_f16x2(folded[i] * il, folded[i + 1] * il), pack_f16x2(folded[i + 2] * il,
                                                                                 folded[i + 3] * il));
      }
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int f = row * NK + i;
        const float il = 1.f / __shfl(l_l, f / VE);
        o[(f / VE) * D + col * VE + (f % VE)] = (uint16_t)(pack_f16x2(folded[i] * il, 0.f) & 0xffffu);
      }
    }
  }

  // Fold the 4 rows: l_l becomes the total of head col; out[i] holds flat accumulator f = row*NK + i.
  __device__ void fold(float* out) {
    l_l = sum_xor32(sum_xor16(l_l));
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
    if (lane < G) { dst[lane] = m_l; dst[G + lane] = l_l; }
  }

  __device__ void write_record(float* __restrict__ rec, const float* folded) const {
    store_ml(rec);
    float* o = rec + rec_ml(G);
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

}  // namespace prr
