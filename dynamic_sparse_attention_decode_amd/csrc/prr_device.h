// prr_device.h — device-side building blocks shared by the PRR kernels (gfx950, wave64).
//
// Token-row layout used by every kernel: one token's key (or value) row is 256 bytes (fp32 x 64 or bf16/fp16 x 128),
// read by 16 lanes with one 16-byte load each, so a wave reads 4 token rows per load instruction: lane = 16*row + col.
// Reductions inside a 16-lane row use DPP; across the 4 rows of a wave they use gfx950's permlane16/32 swaps.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

enum DType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

constexpr int kRowBytes = 256;   // bytes of one token row (head_dim * element size)
constexpr int kRowLanes = 16;    // lanes per token row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- 16-byte vectors of storage elements ------------------------------------------------------------------------

template <int DT> struct Vec;

template <> struct Vec<kF32> {
  static constexpr int n = 4;
  __device__ static inline void to_f32(const uint4 v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static inline uint4 from_f32(const float* o) {   // exact for values that came from storage
    return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
  }
};

template <> struct Vec<kBF16> {
  static constexpr int n = 8;
  __device__ static inline void to_f32(const uint4 v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline uint4 from_f32(const float* o) {   // exact: the low 16 bits are zero
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (__float_as_uint(o[2 * i]) >> 16) | (__float_as_uint(o[2 * i + 1]) & 0xffff0000u);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <> struct Vec<kF16> {
  static constexpr int n = 8;
  __device__ static inline void to_f32(const uint4 v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t h = __builtin_bit_cast(half2_t, w[i]);
      o[2 * i] = (float)h[0];
      o[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static inline uint4 from_f32(const float* o) {   // exact: the values came from fp16 storage
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h;
      h[0] = (_Float16)o[2 * i];
      h[1] = (_Float16)o[2 * i + 1];
      w[i] = __builtin_bit_cast(uint32_t, h);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Two fp32 values as packed fp16 (the conversion rounds to nearest even), and four packed fp16 widened to fp32.
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  half2_t h;
  h[0] = (_Float16)lo;
  h[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, h);
}
__device__ inline float4 unpack_f16x4(uint2 u) {
  const half2_t a = __builtin_bit_cast(half2_t, u.x), b = __builtin_bit_cast(half2_t, u.y);
  return make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
}

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load of data that one step reads once (block summaries, the KV of selected and predicted blocks): a
// non-temporal load, which streams through the caches instead of displacing reused lines. Measured on MI355X, a
// workgroup-contiguous streaming read reaches about 7.0 TB/s with it against 6.2 TB/s with ordinary loads.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// ---- DPP lane exchange inside 16-lane rows -----------------------------------------------------------------------
// dpp_ctrl encodings (GFX9 DPP): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E; row_shl:n = 0x100+n; row_shr:n = 0x110+n;
// row_ror:n = 0x120+n.

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ inline float dpp_f(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROW_MASK,
                                                    BANK_MASK, false));
}

__device__ inline float lane_xor1(float x) { return dpp_f<0xB1>(x, x); }
__device__ inline float lane_xor2(float x) { return dpp_f<0x4E>(x, x); }
// xor 4: banks 0 and 2 (lanes 0-3, 8-11 of a row) take lane+4 (row_shl:4), banks 1 and 3 take lane-4 (row_shr:4)
__device__ inline float lane_xor4(float x) {
  const float t = dpp_f<0x104, 0xF, 0x5>(x, x);
  return dpp_f<0x114, 0xF, 0xA>(t, x);
}
__device__ inline float lane_xor8(float x) { return dpp_f<0x128>(x, x); }   // row_ror:8

__device__ inline float row_sum16(float x) {
  x += lane_xor8(x);
  x += lane_xor4(x);
  x += lane_xor2(x);
  x += lane_xor1(x);
  return x;
}
__device__ inline float row_max16(float x) {
  x = fmaxf(x, lane_xor8(x));
  x = fmaxf(x, lane_xor4(x));
  x = fmaxf(x, lane_xor2(x));
  x = fmaxf(x, lane_xor1(x));
  return x;
}

// ---- exchanges across the rows of a wave (gfx950 v_permlane16_swap / v_permlane32_swap) --------------------------
// swap16(a, b): for each pair of rows (2i, 2i+1) the odd row of `a` and the even row of `b` trade places. With both
// results summed, every lane gets its own value plus its xor-16 partner's. swap32 is the same across the two halves.

struct Pair { float a, b; };

__device__ inline Pair swap16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(a), __float_as_int(b), false, false);
  return {__int_as_float(r[0]), __int_as_float(r[1])};
}
__device__ inline Pair swap32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false);
  return {__int_as_float(r[0]), __int_as_float(r[1])};
}

__device__ inline float sum_xor16(float x) { const Pair p = swap16(x, x); return p.a + p.b; }
__device__ inline float sum_xor32(float x) { const Pair p = swap32(x, x); return p.a + p.b; }
__device__ inline float max_xor16(float x) { const Pair p = swap16(x, x); return fmaxf(p.a, p.b); }
__device__ inline float max_xor32(float x) { const Pair p = swap32(x, x); return fmaxf(p.a, p.b); }

__device__ inline float wave_sum(float x) { return sum_xor32(sum_xor16(row_sum16(x))); }
__device__ inline float wave_max(float x) { return max_xor32(max_xor16(row_max16(x))); }

// Transposing pair reduction across the wave halves: lanes < 32 end with lo(own) + lo(partner), lanes >= 32 with
// hi(own) + hi(partner). One swap reduces two values.
__device__ inline float fold32(float lo, float hi) { const Pair p = swap32(lo, hi); return p.a + p.b; }
// Same across the odd/even rows of each half: even rows keep lo, odd rows keep hi.
__device__ inline float fold16(float lo, float hi) { const Pair p = swap16(lo, hi); return p.a + p.b; }

// ---- order-preserving float -> uint32 keys (larger float -> larger key) -----------------------------------------
// -0 and +0 are one value and take one key (+0's), so equal scores tie by index whatever their sign bit.
__device__ inline uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace prr
