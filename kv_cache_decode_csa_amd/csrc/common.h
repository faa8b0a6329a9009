// Device helpers shared by the HIP kernels of libcsa (gfx950 / CDNA4).
//
// Number formats follow the row layouts of the V4-Flash model record and the
// V4.1-Flash diagram page: OCP E4M3FN values with an E8M0 (power-of-two)
// scale per 32 values, and E2M1 values with an E4M3 scale per 16 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa_internal.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
// Native 4 x u32 vector: unlike HIP's uint4 (a union-wrapped struct) its
// copies stay in registers.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- block cache
// Pool row of logical entry e of sequence b through a block table, or -1 when
// the block id is -1 or outside the pool.  e must lie below max_blocks << shift.
__device__ __forceinline__ int64_t paged_row(const PageMap& m, int64_t b, int64_t e) {
  const int32_t blk = m.table[b * m.max_blocks + (e >> m.shift)];
  return (blk >= 0 && blk < m.pool_blocks)
             ? ((int64_t)blk << m.shift) + (e & (((int64_t)1 << m.shift) - 1))
             : -1;
}

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats -> packed bf16 pair (low half = a)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// exact truncating pack, for values already representable in bf16
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// 2**e as a float for e in [-127, 127] (2**-127 is a float subnormal)
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------- e4m3 (OCP E4M3FN)
// code -> value: placing the 7 magnitude bits under an fp16 exponent of the
// same width plus one gives exactly value / 2**8 for normals and subnormals.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  c &= 0xffu;
  if ((c & 0x7fu) == 0x7fu) return __uint_as_float(0x7fc00000u | ((c & 0x80u) << 24));
  uint16_t h = (uint16_t)(((c & 0x80u) << 8) | ((c & 0x7fu) << 7));
  _Float16 hv = __builtin_bit_cast(_Float16, h);
  return (float)hv * 256.0f;
}

// value -> code, round to nearest even, saturate at +-448; NaN/Inf -> NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return sign | 0x7fu;
  float af = __uint_as_float(a);
  if (af < 0.015625f) {  // below 2**-6: multiples of 2**-9
    uint32_t k = (uint32_t)__builtin_rintf(af * 512.0f);
    return sign | k;  // k == 8 is the smallest normal, code 0x08
  }
  int E = (int)(a >> 23) - 127;
  uint32_t m = a & 0x7fffffu;
  uint32_t r = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;  // RNE to 3 fraction bits
  if (r == 8u) { E += 1; r = 0; }
  if (E > 8 || (E == 8 && r == 7u)) return sign | 0x7eu;
  return sign | ((uint32_t)(E + 7) << 3) | r;
}

// smallest e with amax <= 448 * 2**e, clamped to [-127, 127]; amax finite >= 0
__device__ __forceinline__ int mx32_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  uint32_t ef = b >> 23;
  if (ef == 0) return -127;  // zero or below 2**-126: clamps
  int E = (int)ef - 127;
  int e = E - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- e2m1
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  float v = m < 4u ? 0.5f * (float)m : (m == 4u ? 2.0f : (m == 5u ? 3.0f : (m == 6u ? 4.0f : 6.0f)));
  return (c & 8u) ? -v : v;
}

// RNE onto {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  float a = __builtin_fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  if (__float_as_uint(v) >> 31) c |= 8u;
  return c;
}

// ---------------------------------------------------------------- group encoders
// FP8-MX32: one 32-value group -> 32 codes + one E8M0 scale byte.  `codes`
// must be 4-byte aligned.  FP4-E4M3/16: one 16-value group -> 8 code bytes +
// one E4M3 scale byte.
__device__ __forceinline__ void encode_fp8_group(const float* v, uint8_t* codes, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float a = __builtin_fabsf(v[j]);
    if (a <= 3.402823466e38f) amax = fmaxf(amax, a);  // finite values only
  }
  int e = mx32_exponent(amax);
  *scale = (uint8_t)(e + 127);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c |= f32_to_e4m3(ldexpf(v[4 * q + j], -e)) << (8 * j);
    w[q] = c;
  }
  // rows of 132 bytes are only 4-byte aligned: store dword by dword
#pragma unroll
  for (int q = 0; q < 8; ++q) ((uint32_t*)codes)[q] = w[q];
}

__device__ __forceinline__ void encode_fp4_group(const float* v, uint8_t* codes, uint8_t* scale) {
  float amax = 0.f;
  bool allfin = true;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float a = __builtin_fabsf(v[j]);
    if (a <= 3.402823466e38f) amax = fmaxf(amax, a); else allfin = false;
  }
  uint32_t sc = allfin ? f32_to_e4m3(__fdiv_rn(amax, 6.0f)) : 0x7fu;
  float sv = e4m3_to_f32(sc);
  uint32_t w0 = 0, w1 = 0;
  if (allfin && sv > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w0 |= f32_to_e2m1(__fdiv_rn(v[j], sv)) << (4 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) w1 |= f32_to_e2m1(__fdiv_rn(v[8 + j], sv)) << (4 * j);
  }
  *scale = (uint8_t)sc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // rows may be only 2-byte aligned
    codes[j] = (uint8_t)(w0 >> (8 * j));
    codes[4 + j] = (uint8_t)(w1 >> (8 * j));
  }
}

// MXFP4-MX32: one 32-value group -> 16 code bytes + one E8M0 scale byte.
// X = floor(log2 amax) - 2 (clamped to [-127, 127], amax 0 -> -127); codes
// RNE(x / 2^X) onto E2M1 (exact power-of-two scaling), saturating at 6; a
// group holding a non-finite value gets scale 0xFF and zero codes.
__device__ __forceinline__ int mx4_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const uint32_t ef = b >> 23;
  if (ef == 0) return -127;  // zero or below 2**-126: clamps
  const int X = (int)ef - 127 - 2;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

__device__ __forceinline__ void encode_fp4mx_group(const float* v, uint8_t* codes,
                                                   uint8_t* scale) {
  float amax = 0.f;
  bool allfin = true;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = __builtin_fabsf(v[j]);
    if (a <= 3.402823466e38f) amax = fmaxf(amax, a); else allfin = false;
  }
  const int X = mx4_exponent(amax);
  *scale = allfin ? (uint8_t)(X + 127) : (uint8_t)0xFF;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // rows are 4-byte aligned
    uint32_t w = 0;
    if (allfin) {
#pragma unroll
      for (int j = 0; j < 8; ++j) w |= f32_to_e2m1(ldexpf(v[8 * q + j], -X)) << (4 * j);
    }
    ((uint32_t*)codes)[q] = w;
  }
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Row exchanges of gfx950 (vector ALU, no LDS round trip).  A row is 16 lanes.
// swap_rows16:   x' = [x.r0, y.r0, x.r2, y.r2],  y' = [x.r1, y.r1, x.r3, y.r3]
// swap_halves32: x' = [x.lo, y.lo],              y' = [x.hi, y.hi]
// (the returned pair is copied to plain integers before it is reinterpreted)
__device__ __forceinline__ void swap_rows16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  const uint32_t a = r[0], b = r[1];
  x = a;
  y = b;
}
__device__ __forceinline__ void swap_halves32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  const uint32_t a = r[0], b = r[1];
  x = a;
  y = b;
}
__device__ __forceinline__ void swap_rows16(float& x, float& y) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = __builtin_bit_cast(uint32_t, y);
  swap_rows16(a, b);
  x = __builtin_bit_cast(float, a);
  y = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ void swap_halves32(float& x, float& y) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = __builtin_bit_cast(uint32_t, y);
  swap_halves32(a, b);
  x = __builtin_bit_cast(float, a);
  y = __builtin_bit_cast(float, b);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of a
// 16 x 16 MFMA result), left in all four: the same values and the same
// pairings as xor shuffles by 16 then 32 (max and + are commutative), with
// row swaps on the vector ALU instead of LDS-crossbar permutes.
__device__ __forceinline__ float col_max4(float v) {
  float a = v, b = v;
  swap_rows16(a, b);   // a, b: this lane's row and its partner row (l ^ 16)
  v = fmaxf(a, b);
  a = v;
  b = v;
  swap_halves32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float col_sum4(float v) {
  float a = v, b = v;
  swap_rows16(a, b);
  v = a + b;
  a = v;
  b = v;
  swap_halves32(a, b);
  return a + b;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes, then the row totals carried up (vector ALU lane moves only).
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// MFMA 16x16x32 bf16: A lane l = row (l%16), k 8*(l/16)..+7; B lane l = col (l%16),
// same k; D lane l holds rows 4*(l/16)+r (r = 0..3), col l%16.
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// order-preserving float -> uint32 key for a descending top-k (-0 == +0, NaN lowest)
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- row stores
// Store element c of a finished row: lanes c .. c+31 (FP8) or c .. c+15 (FP4)
// of one group are consecutive lanes of a wave, so the group's amax is a
// shuffle reduction and every lane encodes its own value (the same per-value
// arithmetic as the one-thread group encoders).  Every lane of the wave must
// call it (values past d are passed as 0 with live = false).
__device__ __forceinline__ void store_elem(int fmt, float v, int c, int d, bool live, uint8_t* row) {
  const float av = __builtin_fabsf(v);
  const bool fin = av <= 3.402823466e38f;
  if (fmt == CSA_MIX576) {
    // V4 mixed row (d = 512): a wave holds one block of 64 dims; blocks 0..6
    // are FP8 with an E8M0 scale each, block 7 (dims 448..511) is bf16
    if (c >= 448) {
      if (live) ((uint16_t*)(row + 448))[c - 448] = f32_to_bf16(v);
      if (live && c >= 504) row[583 + (c - 504)] = 0;  // bytes 583..591 stay zero
      if (live && c == 511) row[591] = 0;
      return;
    }
    float amax = fin ? av : 0.f;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    const int e = mx32_exponent(amax);
    const uint32_t code = f32_to_e4m3(ldexpf(v, -e));
    const uint32_t c1 = __shfl_down(code, 1, 64), c2 = __shfl_down(code, 2, 64),
                   c3 = __shfl_down(code, 3, 64);
    if (live && (c & 3) == 0) *(uint32_t*)(row + c) = code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    if (live && (c & 63) == 0) row[576 + (c >> 6)] = (uint8_t)(e + 127);
    return;
  }
  if (fmt == CSA_FP8_MX32) {
    float amax = fin ? av : 0.f;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    const int e = mx32_exponent(amax);
    const uint32_t code = f32_to_e4m3(ldexpf(v, -e));
    // gather 4 codes into the lane holding the first one (rows are 4-byte aligned)
    const uint32_t c1 = __shfl_down(code, 1, 64), c2 = __shfl_down(code, 2, 64),
                   c3 = __shfl_down(code, 3, 64);
    if (live && (c & 3) == 0) *(uint32_t*)(row + c) = code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    if (live && (c & 31) == 0) row[d + (c >> 5)] = (uint8_t)(e + 127);
  } else if (fmt == CSA_FP4_MX32) {
    float amax = fin ? av : 0.f;
    float bad = fin ? 0.f : 1.f;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      amax = fmaxf(amax, shfl_xor_f(amax, m));
      bad = fmaxf(bad, shfl_xor_f(bad, m));
    }
    const bool allfin = bad == 0.f;
    const int X = mx4_exponent(amax);
    const uint32_t code = allfin ? f32_to_e2m1(ldexpf(v, -X)) : 0u;
    const uint32_t odd = __shfl_down(code, 1, 64);
    if (live && (c & 1) == 0) row[c >> 1] = (uint8_t)(code | (odd << 4));
    if (live && (c & 31) == 0) row[d / 2 + (c >> 5)] = allfin ? (uint8_t)(X + 127) : (uint8_t)0xFF;
  } else {
    float amax = fin ? av : 0.f;
    float bad = fin ? 0.f : 1.f;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      amax = fmaxf(amax, shfl_xor_f(amax, m));
      bad = fmaxf(bad, shfl_xor_f(bad, m));
    }
    const bool allfin = bad == 0.f;
    const uint32_t sc = allfin ? f32_to_e4m3(__fdiv_rn(amax, 6.0f)) : 0x7fu;
    const float sv = e4m3_to_f32(sc);
    const uint32_t code = (allfin && sv > 0.f) ? f32_to_e2m1(__fdiv_rn(v, sv)) : 0u;
    const uint32_t odd = __shfl_down(code, 1, 64);
    if (live && (c & 1) == 0) row[c >> 1] = (uint8_t)(code | (odd << 4));
    if (live && (c & 15) == 0) row[d / 2 + (c >> 4)] = (uint8_t)sc;
  }
}

}  // namespace csa
