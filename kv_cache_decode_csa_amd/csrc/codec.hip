// Cache-row codecs and the RoPE table.
//
// Row layouts: FP8-MX32 = dim OCP-E4M3FN codes then dim/32 E8M0 scale bytes
// (the 528-byte decode row of the V4-Flash model record); FP4-E4M3/16 = dim/2
// bytes of E2M1 pairs (element 2j low nibble) then dim/16 E4M3 scales (the
// MXFP4 main-KV format of the V4.1-Flash diagram page, 288 bytes at dim 512).
#include "common.h"

namespace csa {

// ---------------------------------------------------------------- RoPE table
struct Omega {
  double w[kRopeDims / 2];
};

__global__ void rope_table_kernel(Omega om, int64_t rows, float* __restrict__ cos_out,
                                  float* __restrict__ sin_out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * 32) return;
  int64_t p = i >> 5;
  int k = (int)(i & 31);
  double ang = (double)p * om.w[k];
  cos_out[i] = (float)cos(ang);
  sin_out[i] = (float)sin(ang);
}

hipError_t launch_rope_table(const double* omega_host, int64_t rows, float* cos_out,
                             float* sin_out, hipStream_t s) {
  Omega om;
  for (int k = 0; k < kRopeDims / 2; ++k) om.w[k] = omega_host[k];
  int64_t n = rows * 32;
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, om, rows,
                     cos_out, sin_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- group encoders
// One thread encodes one 32-value group (FP8) or one 16-value group (FP4).
__device__ __forceinline__ float load_val(const void* src, int fmt, int64_t i) {
  return fmt == CSA_F32 ? ((const float*)src)[i] : bf16_to_f32(((const uint16_t*)src)[i]);
}

__device__ __forceinline__ void decode_fp8_group(const uint8_t* codes, uint8_t scale, float* v) {
  float f = exp2i((int)scale - 127);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) w[q] = ((const uint32_t*)codes)[q];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * q + j] = e4m3_to_f32(w[q] >> (8 * j)) * f;
}

__device__ __forceinline__ void decode_fp4mx_group(const uint8_t* codes, uint8_t scale, float* v) {
  const float sv = scale == 0xFFu ? __uint_as_float(0x7fc00000u) : exp2i((int)scale - 127);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t b = codes[j];
    v[2 * j] = e2m1_to_f32(b & 15u) * sv;
    v[2 * j + 1] = e2m1_to_f32(b >> 4) * sv;
  }
}

__device__ __forceinline__ void decode_fp4_group(const uint8_t* codes, uint8_t scale, float* v) {
  float sv = e4m3_to_f32(scale);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t b = codes[j];
    v[2 * j] = e2m1_to_f32(b & 15u) * sv;
    v[2 * j + 1] = e2m1_to_f32(b >> 4) * sv;
  }
}

// ---------------------------------------------------------------- kernels
__global__ void quantize_kernel(const void* __restrict__ src, int src_fmt, uint8_t* __restrict__ dst,
                                int dst_fmt, int64_t rows, int dim) {
  const int gsz = dst_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  const int64_t gpr = dim / gsz;
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (dst_fmt == CSA_F32 || dst_fmt == CSA_BF16) {
    // plain cast: one thread per 32 values
    int64_t per = dim / 32;
    if (g >= rows * per) return;
    int64_t base = g * 32;
    for (int j = 0; j < 32; ++j) {
      float x = load_val(src, src_fmt, base + j);
      if (dst_fmt == CSA_F32) ((float*)dst)[base + j] = x;
      else ((uint16_t*)dst)[base + j] = f32_to_bf16(x);
    }
    return;
  }
  if (g >= rows * gpr) return;
  int64_t r = g / gpr;
  int gi = (int)(g % gpr);
  float v[32];
  for (int j = 0; j < gsz; ++j) v[j] = load_val(src, src_fmt, r * dim + (int64_t)gi * gsz + j);
  size_t rb = dst_fmt == CSA_FP8_MX32   ? (size_t)dim + dim / 32
             : dst_fmt == CSA_FP4_MX32 ? (size_t)dim / 2 + dim / 32
                                       : (size_t)dim / 2 + dim / 16;
  uint8_t* row = dst + r * rb;
  if (dst_fmt == CSA_FP8_MX32) encode_fp8_group(v, row + gi * 32, row + dim + gi);
  else if (dst_fmt == CSA_FP4_MX32) encode_fp4mx_group(v, row + gi * 16, row + dim / 2 + gi);
  else encode_fp4_group(v, row + gi * 8, row + dim / 2 + gi);
}

__global__ void dequantize_kernel(const uint8_t* __restrict__ src, int src_fmt, void* __restrict__ dst,
                                  int dst_fmt, int64_t rows, int dim) {
  const int gsz = src_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  const int64_t gpr = dim / gsz;
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * gpr) return;
  int64_t r = g / gpr;
  int gi = (int)(g % gpr);
  float v[32];
  if (src_fmt == CSA_F32) {
    for (int j = 0; j < 32; ++j) v[j] = ((const float*)src)[r * dim + gi * 32 + j];
  } else if (src_fmt == CSA_BF16) {
    for (int j = 0; j < 32; ++j) v[j] = bf16_to_f32(((const uint16_t*)src)[r * dim + gi * 32 + j]);
  } else if (src_fmt == CSA_FP8_MX32) {
    const uint8_t* row = src + r * ((size_t)dim + dim / 32);
    decode_fp8_group(row + gi * 32, row[dim + gi], v);
  } else if (src_fmt == CSA_FP4_MX32) {
    const uint8_t* row = src + r * ((size_t)dim / 2 + dim / 32);
    decode_fp4mx_group(row + gi * 16, row[dim / 2 + gi], v);
  } else {
    const uint8_t* row = src + r * ((size_t)dim / 2 + dim / 16);
    decode_fp4_group(row + gi * 8, row[dim / 2 + gi], v);
  }
  int64_t base = r * dim + (int64_t)gi * gsz;
  for (int j = 0; j < gsz; ++j) {
    if (dst_fmt == CSA_F32) ((float*)dst)[base + j] = v[j];
    else ((uint16_t*)dst)[base + j] = f32_to_bf16(v[j]);
  }
}

// V4 mixed rows (dim 512): bytes [0, 448) E4M3 codes of dims 0..447, [448, 576)
// bf16 dims 448..511, [576, 583) one E8M0 scale per 64 codes, [583, 592) zero.
// One thread per (row, block of 64): blocks 0..6 are FP8, block 7 the bf16 tail.
constexpr int kMixRow = 592;
__global__ void quantize_mix_kernel(const void* __restrict__ src, int src_fmt,
                                    uint8_t* __restrict__ dst, int64_t rows) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * 8) return;
  const int64_t r = g >> 3;
  const int blk = (int)(g & 7);
  uint8_t* row = dst + r * kMixRow;
  const int64_t base = r * 512 + 64 * blk;
  if (blk == 7) {
    for (int j = 0; j < 64; ++j)
      ((uint16_t*)(row + 448))[j] = f32_to_bf16(load_val(src, src_fmt, base + j));
    for (int j = 583; j < kMixRow; ++j) row[j] = 0;
    return;
  }
  float amax = 0.f;
  for (int j = 0; j < 64; ++j) {
    const float a = __builtin_fabsf(load_val(src, src_fmt, base + j));
    if (a <= 3.402823466e38f) amax = fmaxf(amax, a);
  }
  const int e = mx32_exponent(amax);
  row[576 + blk] = (uint8_t)(e + 127);
  for (int q = 0; q < 16; ++q) {
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j)
      w |= f32_to_e4m3(ldexpf(load_val(src, src_fmt, base + 4 * q + j), -e)) << (8 * j);
    ((uint32_t*)(row + 64 * blk))[q] = w;
  }
}

__global__ void dequantize_mix_kernel(const uint8_t* __restrict__ src, void* __restrict__ dst,
                                      int dst_fmt, int64_t rows) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * 8) return;
  const int64_t r = g >> 3;
  const int blk = (int)(g & 7);
  const uint8_t* row = src + r * kMixRow;
  const int64_t base = r * 512 + 64 * blk;
  const float f = blk < 7 ? exp2i((int)row[576 + blk] - 127) : 1.f;
  for (int j = 0; j < 64; ++j) {
    const float v = blk == 7 ? bf16_to_f32(((const uint16_t*)(row + 448))[j])
                             : e4m3_to_f32(row[64 * blk + j]) * f;
    if (dst_fmt == CSA_F32) ((float*)dst)[base + j] = v;
    else ((uint16_t*)dst)[base + j] = f32_to_bf16(v);
  }
}

hipError_t launch_quantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                           int dim, hipStream_t s) {
  if (dst_fmt == CSA_MIX576) {
    hipLaunchKernelGGL(quantize_mix_kernel, dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0,
                       s, src, src_fmt, (uint8_t*)dst, rows);
    return hipGetLastError();
  }
  int gsz = dst_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  int64_t n = rows * (dim / gsz);
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, src_fmt,
                     (uint8_t*)dst, dst_fmt, rows, dim);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                             int dim, hipStream_t s) {
  if (src_fmt == CSA_MIX576) {
    hipLaunchKernelGGL(dequantize_mix_kernel, dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256),
                       0, s, (const uint8_t*)src, dst, dst_fmt, rows);
    return hipGetLastError();
  }
  int gsz = src_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  int64_t n = rows * (dim / gsz);
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint8_t*)src, src_fmt, dst, dst_fmt, rows, dim);
  return hipGetLastError();
}

}  // namespace csa
