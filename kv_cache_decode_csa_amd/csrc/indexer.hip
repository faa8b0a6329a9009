// Lightning-indexer scores ("DeepSeek-V4 deep dive" section 5.2):
//   score[s] = sum_h w_h * ReLU(q_h . k_s),   s < n_vis = min(floor((pos+1)/ratio), Nmax)
// The key stream is the dominant HBM traffic of a CSA decode step at long
// context, so the kernel reads every key once, coalesced, and does the
// heads x 128 contraction on MFMA (bf16 operands, float32 accumulation).
// FP8-MX32 keys (132 B: 128 E4M3 codes + 4 E8M0 scales) are decoded exactly to
// bf16 in registers; one MFMA k-step covers 32 dims, i.e. exactly one scale
// group.  The epilogue applies ReLU and the head weights, reduces over heads,
// writes the score and adds its top-k radix digit to a row histogram.
#include "common.h"

namespace csa {

namespace {

constexpr int kIdxThreads = 256;
constexpr int kKeysPerWave = 16;
constexpr int kIters = 16;                                     // 16-key groups per wave
constexpr int kKeysPerWg = kKeysPerWave * 4 * kIters;          // 1024

// 8 E4M3 codes (two dwords) times 2**e -> 8 exact bf16 values
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi, float scale) {
  uint4 r;
  r.x = pack_bf16x2_exact(e4m3_to_f32(lo) * scale, e4m3_to_f32(lo >> 8) * scale);
  r.y = pack_bf16x2_exact(e4m3_to_f32(lo >> 16) * scale, e4m3_to_f32(lo >> 24) * scale);
  r.z = pack_bf16x2_exact(e4m3_to_f32(hi) * scale, e4m3_to_f32(hi >> 8) * scale);
  r.w = pack_bf16x2_exact(e4m3_to_f32(hi >> 16) * scale, e4m3_to_f32(hi >> 24) * scale);
  return r;
}

template <int HT, int KFMT>
__global__ void __launch_bounds__(kIdxThreads) index_scores_mfma(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores, int32_t* __restrict__ n_vis_out,
    uint32_t* __restrict__ hist_g) {
  constexpr int Hi = HT * 16;
  constexpr int64_t kRowBytes = KFMT == CSA_FP8_MX32 ? 132 : 256;
  __shared__ uint32_t hist[kHistBins];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t row = row_off + blockIdx.y;  // b * Q + q
  const int64_t b = row / Q;
  int64_t nv = ((int64_t)pos[row] + 1) / ratio;
  nv = nv < 0 ? 0 : (nv > Nmax ? Nmax : nv);
  if (blockIdx.x == 0 && t == 0) n_vis_out[row] = (int32_t)nv;
  const int64_t base = (int64_t)blockIdx.x * kKeysPerWg;
  if (base >= nv) return;

  for (int i = t; i < kHistBins; i += kIdxThreads) hist[i] = 0;

  // query fragments (MFMA A operand): head 16*mt + lane%16, dims 32*s + 8*(lane/16) .. +8
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  uint4 qa[HT][4];
  const uint16_t* qrow = q_idx + row * (int64_t)Hi * kIndexDim;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[mt][s] = *(const uint4*)(qrow + (16 * mt + r16) * kIndexDim + 32 * s + 8 * kq);
  // head weights for the D layout: head 16*mt + 4*(lane/16) + r
  float wv[HT][4];
  const float* wrow = w_idx + row * (int64_t)Hi;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wrow[16 * mt + 4 * kq + r];
  __syncthreads();

  const uint8_t* kbase = k_idx + b * Nmax * kRowBytes;
  float* srow = scores + row * Nmax;

  for (int it = 0; it < kIters; ++it) {
    const int64_t key0 = base + (int64_t)kKeysPerWave * (wave + 4 * it);
    if (key0 >= nv) break;
    const int64_t key = key0 + r16;
    const bool valid = key < nv;
    uint4 kb[4];
    if (KFMT == CSA_FP8_MX32) {
      const uint8_t* kr = kbase + key * kRowBytes;
      uint32_t lo[4], hi[4], sc = 0;
      if (valid) {
        sc = *(const uint32_t*)(kr + 128);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          lo[s] = *(const uint32_t*)(kr + 32 * s + 8 * kq);
          hi[s] = *(const uint32_t*)(kr + 32 * s + 8 * kq + 4);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) lo[s] = hi[s] = 0;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kb[s] = fp8x8_to_bf16x8(lo[s], hi[s], exp2i((int)((sc >> (8 * s)) & 0xffu) - 127));
    } else {
      const uint16_t* kr = (const uint16_t*)(kbase + key * kRowBytes);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kb[s] = valid ? *(const uint4*)(kr + 32 * s + 8 * kq) : make_uint4(0, 0, 0, 0);
    }
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as_bf16x8(qa[mt][s]), as_bf16x8(kb[s]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) p += wv[mt][r] * fmaxf(acc[r], 0.f);
    }
    p += shfl_xor_f(p, 16);
    p += shfl_xor_f(p, 32);
    if (kq == 0 && valid) {
      srow[key] = p;
      atomicAdd(&hist[score_key(p) >> 20], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = hist_g + row * kHistBins;
  for (int i = t; i < kHistBins; i += kIdxThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// float32 path: one thread per key, q in LDS.
constexpr int kF32Keys = 256;
__global__ void __launch_bounds__(kIdxThreads) index_scores_f32(
    const float* __restrict__ q_idx, const float* __restrict__ w_idx,
    const float* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q, int Hi,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores, int32_t* __restrict__ n_vis_out,
    uint32_t* __restrict__ hist_g) {
  __shared__ float qs[128 * kIndexDim];
  __shared__ float ws[128];
  __shared__ uint32_t hist[kHistBins];
  const int t = threadIdx.x;
  const int64_t row = row_off + blockIdx.y;
  const int64_t b = row / Q;
  int64_t nv = ((int64_t)pos[row] + 1) / ratio;
  nv = nv < 0 ? 0 : (nv > Nmax ? Nmax : nv);
  if (blockIdx.x == 0 && t == 0) n_vis_out[row] = (int32_t)nv;
  const int64_t base = (int64_t)blockIdx.x * kF32Keys;
  if (base >= nv) return;
  for (int i = t; i < kHistBins; i += kIdxThreads) hist[i] = 0;
  for (int i = t; i < Hi * kIndexDim; i += kIdxThreads) qs[i] = q_idx[row * Hi * kIndexDim + i];
  for (int i = t; i < Hi; i += kIdxThreads) ws[i] = w_idx[row * Hi + i];
  __syncthreads();
  const int64_t key = base + t;
  if (key < nv) {
    const float* kr = k_idx + (b * Nmax + key) * kIndexDim;
    float kv[kIndexDim];
#pragma unroll
    for (int c = 0; c < kIndexDim; ++c) kv[c] = kr[c];
    float p = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < kIndexDim; ++c) d = fmaf(qs[h * kIndexDim + c], kv[c], d);
      p = fmaf(ws[h], fmaxf(d, 0.f), p);
    }
    scores[row * Nmax + key] = p;
    atomicAdd(&hist[score_key(p) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* g = hist_g + row * kHistBins;
  for (int i = t; i < kHistBins; i += kIdxThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

template <int HT>
hipError_t launch_mfma(const void* q_idx, const float* w_idx, const void* k_idx, int k_fmt,
                       const int32_t* pos, int ratio, int Q, int64_t R, int64_t Nmax,
                       float* scores, int32_t* n_vis, uint32_t* hist, hipStream_t s) {
  int64_t gx = (Nmax + kKeysPerWg - 1) / kKeysPerWg;
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    if (k_fmt == CSA_FP8_MX32)
      hipLaunchKernelGGL((index_scores_mfma<HT, CSA_FP8_MX32>), dim3((unsigned)gx, (unsigned)nr),
                         dim3(kIdxThreads), 0, s, (const uint16_t*)q_idx, w_idx,
                         (const uint8_t*)k_idx, pos, ratio, Q, Nmax, r0, scores, n_vis, hist);
    else
      hipLaunchKernelGGL((index_scores_mfma<HT, CSA_BF16>), dim3((unsigned)gx, (unsigned)nr),
                         dim3(kIdxThreads), 0, s, (const uint16_t*)q_idx, w_idx,
                         (const uint8_t*)k_idx, pos, ratio, Q, Nmax, r0, scores, n_vis, hist);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const void* q_idx, int q_fmt, const float* w_idx,
                               const void* k_idx, int k_fmt, const int32_t* pos, int ratio, int B,
                               int Q, int Hi, int64_t Nmax, float* scores, int32_t* n_vis,
                               TopkWs w, hipStream_t s) {
  const int64_t R = (int64_t)B * Q;
  if (k_fmt == CSA_F32) {
    int64_t gx = (Nmax + kF32Keys - 1) / kF32Keys;
    for (int64_t r0 = 0; r0 < R; r0 += 65535) {
      int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
      hipLaunchKernelGGL(index_scores_f32, dim3((unsigned)gx, (unsigned)nr), dim3(kIdxThreads), 0,
                         s, (const float*)q_idx, w_idx, (const float*)k_idx, pos, ratio, Q, Hi,
                         Nmax, r0, scores, n_vis, w.hist);
    }
    return hipGetLastError();
  }
  (void)q_fmt;
  switch (Hi / 16) {
    case 1: return launch_mfma<1>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 2: return launch_mfma<2>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 3: return launch_mfma<3>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 4: return launch_mfma<4>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 5: return launch_mfma<5>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 6: return launch_mfma<6>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 7: return launch_mfma<7>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    case 8: return launch_mfma<8>(q_idx, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
