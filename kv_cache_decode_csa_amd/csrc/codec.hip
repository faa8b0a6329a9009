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

hipError_t launch_quantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                           int dim, hipStream_t s) {
  int gsz = dst_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  int64_t n = rows * (dim / gsz);
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, src_fmt,
                     (uint8_t*)dst, dst_fmt, rows, dim);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                             int dim, hipStream_t s) {
  int gsz = src_fmt == CSA_FP4_E4M3_16 ? 16 : 32;
  int64_t n = rows * (dim / gsz);
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint8_t*)src, src_fmt, dst, dst_fmt, rows, dim);
  return hipGetLastError();
}

}  // namespace csa
