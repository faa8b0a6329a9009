// Learned gated-pooling compressor ("DeepSeek-V4 deep dive" sections 4.1-4.3,
// and the indexer's 128-wide rotated compressor of section 5.2).
//
// Three kernels, in stream order:
//   1. projection   P[b, i] = [W_kv x ; W_gate x] for every token of the call
//      (float32 out; a weight-streaming GEMV when B*T is small, a tiled GEMM
//      otherwise);
//   2. emit         one work-group per block completed by the call: gathers the
//      block's slots (from P for tokens of this call, from the slot state for
//      earlier tokens), pools every channel with a softmax over the slots,
//      RMSNorm -> RoPE at the block's first position -> optional Hadamard ->
//      storage rounding, and writes the entry;
//   3. state        one thread per state column rewrites all slots of that
//      column (reads first, then writes, so the overlap shift is race-free).
#include "common.h"

namespace csa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float ldv(const void* p, int fmt, int64_t i) {
  return fmt == CSA_F32 ? ((const float*)p)[i] : bf16_to_f32(((const uint16_t*)p)[i]);
}

// ------------------------------------------------------------------ projection
// GEMV for M = B*T <= 16: each wave produces two output columns for all rows.
constexpr int kGemvMaxM = 16;

__global__ void __launch_bounds__(kThreads) proj_gemv_kernel(const void* __restrict__ x, int x_fmt,
                                                             const void* __restrict__ wkv,
                                                             const void* __restrict__ wg,
                                                             int w_fmt, int M, int K, int CD,
                                                             float* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = 2 * CD;
  const int n0 = (blockIdx.x * 4 + wave) * 2;
  float acc[2][kGemvMaxM];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < kGemvMaxM; ++m) acc[c][m] = 0.f;
  for (int k = 8 * lane; k < K; k += 512) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int n = n0 + c;
      if (n >= N) break;
      const void* W = n < CD ? wkv : wg;
      const int64_t wr = (int64_t)(n < CD ? n : n - CD) * K + k;
      float wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = ldv(W, w_fmt, wr + j);
#pragma unroll
      for (int m = 0; m < kGemvMaxM; ++m) {
        if (m >= M) break;
        float s = acc[c][m];
#pragma unroll
        for (int j = 0; j < 8; ++j) s = fmaf(wv[j], ldv(x, x_fmt, (int64_t)m * K + k + j), s);
        acc[c][m] = s;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int n = n0 + c;
#pragma unroll
    for (int m = 0; m < kGemvMaxM; ++m) {
      if (m >= M) break;
      float v = wave_sum(acc[c][m]);
      if (lane == 0 && n < N) P[(int64_t)m * N + n] = v;
    }
  }
}

// Tiled GEMM, float32 FMA: P[m][n] = sum_k x[m][k] W[n][k], 64x64 tiles.
constexpr int kTM = 64, kTN = 64, kTK = 32;

__global__ void __launch_bounds__(kThreads) proj_gemm_kernel(const void* __restrict__ x, int x_fmt,
                                                             const void* __restrict__ wkv,
                                                             const void* __restrict__ wg,
                                                             int w_fmt, int64_t M, int K, int CD,
                                                             float* __restrict__ P) {
  __shared__ float Xs[kTK][kTM + 1];
  __shared__ float Ws[kTK][kTN + 1];
  const int tid = threadIdx.x;
  const int N = 2 * CD;
  const int64_t m0 = (int64_t)blockIdx.y * kTM;
  const int n0 = blockIdx.x * kTN;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kTK) {
    for (int i = tid; i < kTM * kTK; i += kThreads) {
      const int r = i / kTK, c = i % kTK;
      const int64_t m = m0 + r;
      const int k = k0 + c;
      Xs[c][r] = (m < M && k < K) ? ldv(x, x_fmt, m * K + k) : 0.f;
      const int n = n0 + r;
      float wv = 0.f;
      if (n < N && k < K) {
        const void* W = n < CD ? wkv : wg;
        wv = ldv(W, w_fmt, (int64_t)(n < CD ? n : n - CD) * K + k);
      }
      Ws[c][r] = wv;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kTK; ++c) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xa[i] = Xs[c][tm + i]; wb[i] = Ws[c][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn + j;
      if (n < N) P[m * N + n] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ shared helpers
struct CompArgs {
  int B, T, ratio, coff, d, CD, rotate, entry_fmt;
  const float* ape;
  const float* norm_w;
  float eps;
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_rows;
  const int32_t* start_pos;
  float* kv_state;
  float* score_state;
  uint8_t* entries;
  int64_t entries_cap;
  size_t entry_rb;
  const float* P;  // [B*T][2*CD]
};

// (v, s) of token p of sequence b at state column col (0 <= col < CD), where
// the call starts at p0.  Tokens before p0 are read from the state as given.
__device__ __forceinline__ void token_vs(const CompArgs& a, int64_t b, int64_t p0, int64_t p,
                                         int col, float& v, float& s) {
  if (p < 0) {
    v = 0.f;
    s = -INFINITY;
    return;
  }
  if (p >= p0) {
    const float* row = a.P + (b * a.T + (p - p0)) * (int64_t)(2 * a.CD);
    v = row[col];
    s = row[a.CD + col] + a.ape[(int64_t)(p % a.ratio) * a.CD + col];
    return;
  }
  const int64_t cur = p0 / a.ratio;
  int slot;
  if (p / a.ratio == cur) slot = (a.coff == 2 ? a.ratio : 0) + (int)(p % a.ratio);
  else slot = (int)(p % a.ratio);  // previous block (overlap only)
  const int64_t si = (b * (int64_t)(a.coff * a.ratio) + slot) * a.CD + col;
  v = a.kv_state[si];
  s = a.score_state[si];
}

// ------------------------------------------------------------------ emit
__global__ void __launch_bounds__(kThreads) emit_kernel(CompArgs a) {
  __shared__ float y[512];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t p0 = a.start_pos[b];
  const int r = a.ratio;
  const int64_t i = p0 / r + blockIdx.x;              // candidate block
  if (p0 < 0 || (i + 1) * r - 1 >= p0 + a.T) return;  // not completed by this call
  const int d = a.d;

  // pool each channel over its slots
  float sq = 0.f;
  for (int c = tid; c < d; c += kThreads) {
    float mx = -INFINITY;
    // first pass: max score
    const int nslots = a.coff * r;
    for (int sl = 0; sl < nslots; ++sl) {
      int64_t p;
      int col;
      if (a.coff == 2) {
        p = sl < r ? (i - 1) * r + sl : i * r + (sl - r);
        col = sl < r ? c : d + c;
      } else {
        p = i * r + sl;
        col = c;
      }
      float v, s;
      token_vs(a, b, p0, p, col, v, s);
      mx = fmaxf(mx, s);
    }
    float num = 0.f, den = 0.f;
    for (int sl = 0; sl < nslots; ++sl) {
      int64_t p;
      int col;
      if (a.coff == 2) {
        p = sl < r ? (i - 1) * r + sl : i * r + (sl - r);
        col = sl < r ? c : d + c;
      } else {
        p = i * r + sl;
        col = c;
      }
      float v, s;
      token_vs(a, b, p0, p, col, v, s);
      const float e = (s == -INFINITY) ? 0.f : expf(s - mx);
      num = fmaf(e, v, num);
      den += e;
    }
    const float C = num / den;
    y[c] = C;
    sq = fmaf(C, C, sq);
  }
  sq = wave_sum(sq);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  const float ms = ((red[0] + red[1]) + (red[2] + red[3])) / (float)d;
  const float inv = 1.0f / sqrtf(ms + a.eps);
  for (int c = tid; c < d; c += kThreads) y[c] = y[c] * inv * a.norm_w[c];
  __syncthreads();
  // RoPE on the last 64 dims at position i * r
  {
    int64_t rrow = i * r;
    if (rrow >= a.rope_rows) rrow = a.rope_rows - 1;
    if (tid < kRopeDims / 2) {
      const int c0 = d - kRopeDims + 2 * tid;
      const float cs = a.rope_cos[rrow * 32 + tid], sn = a.rope_sin[rrow * 32 + tid];
      const float x0 = y[c0], x1 = y[c0 + 1];
      y[c0] = x0 * cs - x1 * sn;
      y[c0 + 1] = x0 * sn + x1 * cs;
    }
    __syncthreads();
  }
  // Sylvester Hadamard (butterflies a+b, a-b at strides 1..d/2), scaled by d^-1/2
  if (a.rotate) {
    for (int h = 1; h < d; h <<= 1) {
      for (int q = tid; q < d / 2; q += kThreads) {
        const int lo = (q / h) * 2 * h + (q % h);
        const float u = y[lo], v = y[lo + h];
        y[lo] = u + v;
        y[lo + h] = u - v;
      }
      __syncthreads();
    }
    const float sc = 1.0f / sqrtf((float)d);
    for (int c = tid; c < d; c += kThreads) y[c] *= sc;
    __syncthreads();
  }
  if (i >= a.entries_cap) return;
  uint8_t* row = a.entries + ((size_t)b * (size_t)a.entries_cap + (size_t)i) * a.entry_rb;
  if (a.entry_fmt == CSA_F32) {
    for (int c = tid; c < d; c += kThreads) ((float*)row)[c] = y[c];
  } else if (a.entry_fmt == CSA_BF16) {
    for (int c = tid; c < d; c += kThreads) ((uint16_t*)row)[c] = f32_to_bf16(y[c]);
  } else if (a.entry_fmt == CSA_FP8_MX32) {
    if (tid < d / 32) encode_fp8_group(y + 32 * tid, row + 32 * tid, row + d + tid);
  } else {
    if (tid < d / 16) encode_fp4_group(y + 16 * tid, row + 8 * tid, row + d / 2 + tid);
  }
}

// ------------------------------------------------------------------ state
// New slot contents after the call, as the token-by-token decode state machine
// leaves them: the unfinished block's tokens in their current slots; if a
// block completed in this call, every other current slot (and, with overlap,
// every previous slot) holds the last completed block.  Slots whose token
// precedes the call keep their value, except the overlap shift, which copies
// current slots into previous ones -- done from values read before any write.
__global__ void __launch_bounds__(kThreads) state_kernel(CompArgs a) {
  const int64_t b = blockIdx.y;
  const int col = blockIdx.x * kThreads + threadIdx.x;
  if (col >= a.CD) return;
  const int64_t p0 = a.start_pos[b];
  if (p0 < 0) return;
  const int r = a.ratio;
  const int64_t p1 = p0 + a.T;
  const int64_t first_block = p0 / r, end_block = p1 / r;
  const int nslots = a.coff * r;
  const int64_t sbase = b * (int64_t)nslots * a.CD + col;
  const int64_t unfinished0 = end_block * r > p0 ? end_block * r : p0;
  if (a.coff == 1) {
    // no slot moves: tokens of this call land in slot p mod r
    for (int64_t p = unfinished0; p < p1; ++p) {
      float v, sc;
      token_vs(a, b, p0, p, col, v, sc);
      a.kv_state[sbase + (p % r) * a.CD] = v;
      a.score_state[sbase + (p % r) * a.CD] = sc;
    }
    if (end_block > first_block) {
      const int64_t done = end_block - 1;
      for (int q = (int)(p1 - end_block * r); q < r; ++q) {
        const int64_t p = done * r + q;
        if (p < p0) continue;  // already in its slot
        float v, sc;
        token_vs(a, b, p0, p, col, v, sc);
        a.kv_state[sbase + (int64_t)q * a.CD] = v;
        a.score_state[sbase + (int64_t)q * a.CD] = sc;
      }
    }
    return;
  }
  // overlap (ratio 4): 8 slots, decide all from the old state, then write
  float nv[8], ns[8];
  bool wr[8];
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) wr[sl] = false;
  for (int64_t p = unfinished0; p < p1; ++p) {
    const int sl = r + (int)(p % r);
    token_vs(a, b, p0, p, col, nv[sl], ns[sl]);
    wr[sl] = true;
  }
  if (end_block > first_block) {
    const int64_t done = end_block - 1;
    for (int q = 0; q < r; ++q) {
      const int64_t p = done * r + q;
      token_vs(a, b, p0, p, col, nv[q], ns[q]);
      wr[q] = true;
      if (!wr[r + q]) {
        nv[r + q] = nv[q];
        ns[r + q] = ns[q];
        wr[r + q] = true;
      }
    }
  }
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    if (!wr[sl]) continue;
    a.kv_state[sbase + (int64_t)sl * a.CD] = nv[sl];
    a.score_state[sbase + (int64_t)sl * a.CD] = ns[sl];
  }
}

}  // namespace

size_t compress_ws_bytes(const csa_compress_args* a) {
  const int coff = a->ratio == 4 ? 2 : 1;
  const int CD = coff * a->head_dim;
  return align_up((size_t)a->B * a->T * 2 * CD * sizeof(float), 256);
}

hipError_t launch_compress(const csa_compress_args* in, void* ws, hipStream_t s) {
  CompArgs a;
  a.B = in->B;
  a.T = in->T;
  a.ratio = in->ratio;
  a.coff = in->ratio == 4 ? 2 : 1;
  a.d = in->head_dim;
  a.CD = a.coff * a.d;
  a.rotate = in->rotate;
  a.entry_fmt = in->entry_fmt;
  a.ape = in->ape;
  a.norm_w = in->norm_w;
  a.eps = in->eps;
  a.rope_cos = in->rope_cos;
  a.rope_sin = in->rope_sin;
  a.rope_rows = in->rope_rows;
  a.start_pos = in->start_pos;
  a.kv_state = in->kv_state;
  a.score_state = in->score_state;
  a.entries = (uint8_t*)in->entries;
  a.entries_cap = in->entries_cap;
  a.entry_rb = kv_row_bytes(in->entry_fmt, in->head_dim);
  float* P = (float*)ws;
  a.P = P;
  const int64_t M = (int64_t)in->B * in->T;
  const int N = 2 * a.CD;
  if (M <= kGemvMaxM) {
    hipLaunchKernelGGL(proj_gemv_kernel, dim3((N + 7) / 8), dim3(kThreads), 0, s, in->x,
                       in->x_fmt, in->w_kv, in->w_gate, in->w_fmt, (int)M, in->dim, a.CD, P);
  } else {
    for (int64_t m0 = 0; m0 < M; m0 += (int64_t)65535 * kTM) {
      const int64_t mm = M - m0 < (int64_t)65535 * kTM ? M - m0 : (int64_t)65535 * kTM;
      const size_t xoff = (size_t)m0 * in->dim * (in->x_fmt == CSA_F32 ? 4 : 2);
      hipLaunchKernelGGL(proj_gemm_kernel, dim3((N + kTN - 1) / kTN, (unsigned)((mm + kTM - 1) / kTM)),
                         dim3(kThreads), 0, s, (const void*)((const char*)in->x + xoff), in->x_fmt,
                         in->w_kv, in->w_gate, in->w_fmt, mm, in->dim, a.CD, P + m0 * N);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int max_blocks = in->T / in->ratio + 1;
  hipLaunchKernelGGL(emit_kernel, dim3(max_blocks, in->B), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(state_kernel, dim3((a.CD + kThreads - 1) / kThreads, in->B), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace csa
