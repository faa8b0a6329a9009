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
constexpr int kEmitT1Threads = 512;  // single-token emit: one channel per thread at d = 512

// Orders one wave's LDS accesses (LDS operations of a wave execute in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// MFMA projection for bf16 x and W with M = B*T <= 64 (decode): each work-group
// streams 16 weight rows over the whole of K with 8 waves, each wave taking
// 1/8 of K in steps of 8 x 32 (eight 16-byte loads in flight per lane).  The
// waves' 16x16 partial products are summed in LDS in a fixed order.  A lane
// holds x[m][k + 8 kq .. +8] (A) and W[n][k + 8 kq .. +8] (B): contiguous
// 16-byte loads.  Single-token calls write the result straight into the slot
// state (score gets its slot bias); otherwise into P[M][N].
constexpr int kMfmaMaxM = 64;
constexpr int kProjThreads = 512;

struct ProjOut {
  float* P;                   // [M][N] when not direct
  int direct;                 // 1: T == 1, write state slots
  const int32_t* start_pos;   // [B]
  const float* ape;           // [ratio][CD]
  int ratio, coff;
  float* kv_state;            // [B][coff*ratio][CD]
  float* score_state;
};

template <int MT>
__global__ void __launch_bounds__(kProjThreads) proj_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wkv,
                                                                 const uint16_t* __restrict__ wg,
                                                                 int M, int K, int CD, ProjOut po) {
  __shared__ f32x4_t red[8][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int N = 2 * CD;
  const int n = blockIdx.x * 16 + r16;
  const uint16_t* wrow = n < CD ? wkv + (int64_t)n * K : wg + (int64_t)(n - CD) * K;
  // epilogue inputs of the direct (single-token) mode, fetched up front: the
  // position of each of this thread's 4 output rows and the score columns'
  // slot bias
  const int tt = threadIdx.x;
  const int emt = tt >> 6, el = tt & 63;
  const int enn = blockIdx.x * 16 + (el & 15);
  int64_t ep[4];
  float eape[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 16 * emt + 4 * (el >> 4) + r;
    ep[r] = -1;
    eape[r] = 0.f;
    if (po.direct && tt < MT * 64 && m < M) {
      ep[r] = po.start_pos[m];
      if (enn >= CD && ep[r] >= 0) eape[r] = po.ape[(ep[r] % po.ratio) * CD + enn - CD];
    }
  }
  // wave w covers k in [w K/8, (w+1) K/8): nks steps of 32.  All of a batch's
  // loads are issued before its MFMAs (addresses clamped to valid steps and
  // rows, out-of-range operands zeroed), so they are in flight together.
  constexpr int kB = MT <= 2 ? 16 : 8;
  const int nks = K / 256;
  const int kb = wave * (K / 8);
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks0 = 0; ks0 < nks; ks0 += kB) {
    u32x4_t bw[kB];
    u32x4_t ax[kB][MT];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int ks = ks0 + u < nks ? ks0 + u : nks - 1;
      const int k = kb + 32 * ks + 8 * kq;
      bw[u] = *(const u32x4_t*)(wrow + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16 < M ? 16 * mt + r16 : M - 1;
        ax[u][mt] = *(const u32x4_t*)(x + (int64_t)m * K + k);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool step_ok = ks0 + u < nks;  // a clamped repeat of the last step adds zero
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t av = (step_ok && 16 * mt + r16 < M) ? ax[u][mt] : u32x4_t{0u, 0u, 0u, 0u};
        acc[mt] = mfma16x16x32(as_bf16x8(av), as_bf16x8(bw[u]), acc[mt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();
  if (tt < MT * 64) {
    const int mt = emt, l = el;
    f32x4_t v = red[0][mt][l];
#pragma unroll
    for (int w = 1; w < 8; ++w) {
      const f32x4_t u = red[w][mt][l];
      v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
    }
    const int nn = enn;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * (l >> 4) + r;
      if (m >= M) continue;
      if (!po.direct) {
        po.P[(int64_t)m * N + nn] = v[r];
        continue;
      }
      const int64_t p = ep[r];
      if (p < 0) continue;
      const int slot = (po.coff == 2 ? po.ratio : 0) + (int)(p % po.ratio);
      const int64_t base = ((int64_t)m * po.coff * po.ratio + slot) * CD;
      if (nn < CD) po.kv_state[base + nn] = v[r];
      else po.score_state[base + nn - CD] = v[r] + eape[r];
    }
  }
}

// Single-token (decode) projection split over K: work-group (column block,
// k slice ks, block of 64 token rows) is one wave that takes 16 weight rows
// over k in [ks K/8, (ks+1) K/8) -- all of its loads in flight together -- and
// writes the 16 x (up to 64) partial products to part[ks][m][n].  The emit
// kernel adds the eight slices in order, the same summation as the
// one-work-group projection above.  Batches of more than 64 tokens take
// several row blocks, each streaming the weights again (through L2 when the
// row blocks of a column block run together).
constexpr int kKSlices = 8;
constexpr int kMaxJobs = 4;       // compressors fused into one launch
constexpr int kSliceRows = 64;    // token rows per work-group
constexpr int kSliceMaxM = 1024;  // larger single-token batches take the tiled GEMM

struct ProjJob {
  const uint16_t* x;    // [M][K] bf16
  const uint16_t* wkv;  // [CD][K]
  const uint16_t* wg;   // [CD][K]
  int K, CD;
  int blk0;             // first column block of this job in the launch
  float* part;          // [kKSlices][M][2 CD]
};
struct ProjJobs {
  ProjJob j[kMaxJobs];
  int n;
};

template <int MT>
__global__ void __launch_bounds__(64) proj_slice_kernel(ProjJobs jobs, int M) {
  int jb = 0;
#pragma unroll
  for (int q = 1; q < kMaxJobs; ++q)
    if (q < jobs.n && (int)blockIdx.x >= jobs.j[q].blk0) jb = q;
  const ProjJob& J = jobs.j[jb];
  const uint16_t* __restrict__ x = J.x;
  const int K = J.K, CD = J.CD;
  const int lane = threadIdx.x;
  const int r16 = lane & 15, kq = lane >> 4;
  const int N = 2 * CD;
  const int cb = (int)blockIdx.x - J.blk0;
  const int n = cb * 16 + r16;
  const int m0 = (int)blockIdx.z * kSliceRows;  // this work-group's token rows
  const uint16_t* wrow = n < CD ? J.wkv + (int64_t)n * K : J.wg + (int64_t)(n - CD) * K;
  constexpr int kB = MT <= 2 ? 16 : 8;
  const int nks = K / 256;
  const int kb = blockIdx.y * (K / kKSlices);
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks0 = 0; ks0 < nks; ks0 += kB) {
    u32x4_t bw[kB];
    u32x4_t ax[kB][MT];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int ks = ks0 + u < nks ? ks0 + u : nks - 1;
      const int k = kb + 32 * ks + 8 * kq;
      bw[u] = *(const u32x4_t*)(wrow + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + r16 < M ? m0 + 16 * mt + r16 : M - 1;
        ax[u][mt] = *(const u32x4_t*)(x + (int64_t)m * K + k);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool step_ok = ks0 + u < nks;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t av = (step_ok && m0 + 16 * mt + r16 < M) ? ax[u][mt] : u32x4_t{0u, 0u, 0u, 0u};
        acc[mt] = mfma16x16x32(as_bf16x8(av), as_bf16x8(bw[u]), acc[mt]);
      }
    }
  }
  float* dst = J.part + (int64_t)blockIdx.y * M * N + cb * 16 + (lane & 15);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mt + 4 * (lane >> 4) + r;
      if (m < M) dst[(int64_t)m * N] = acc[mt][r];
    }
}

// The same products for batches of more than 64 tokens: one wave per (64
// output columns, K/8 slice, 64 token rows) with 4 x 4 MFMA tiles per k-step,
// so each x fragment it loads serves four column tiles (a quarter of the x
// reads of the 16-column form).  Every output takes the same MFMA steps in
// the same order as in proj_slice_kernel, so the two give the same bits.
// Job column blocks (blk0) count 64-column blocks here (2 CD is a multiple of
// 64: head dims are 128 or 512).
__global__ void __launch_bounds__(64) proj_slice_wide_kernel(ProjJobs jobs, int M) {
  int jb = 0;
#pragma unroll
  for (int q = 1; q < kMaxJobs; ++q)
    if (q < jobs.n && (int)blockIdx.x >= jobs.j[q].blk0) jb = q;
  const ProjJob& J = jobs.j[jb];
  const int K = J.K, CD = J.CD;
  const int N = 2 * CD;
  const int lane = threadIdx.x;
  const int r16 = lane & 15, kq = lane >> 4;
  const int cb = (int)blockIdx.x - J.blk0;      // 64-column block
  const int m0 = (int)blockIdx.z * kSliceRows;  // this work-group's token rows
  const uint16_t* wrow[4];
  const uint16_t* xrow[4];
  bool mok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = 64 * cb + 16 * t + r16;
    wrow[t] = n < CD ? J.wkv + (int64_t)n * K : J.wg + (int64_t)(n - CD) * K;
    const int m = m0 + 16 * t + r16;
    mok[t] = m < M;
    xrow[t] = J.x + (int64_t)(m < M ? m : M - 1) * K;
  }
  constexpr int kB = 4;
  const int nks = K / 256;
  const int kb = blockIdx.y * (K / kKSlices);
  f32x4_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks0 = 0; ks0 < nks; ks0 += kB) {
    u32x4_t bw[kB][4], ax[kB][4];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int ks = ks0 + u < nks ? ks0 + u : nks - 1;
      const int k = kb + 32 * ks + 8 * kq;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bw[u][t] = *(const u32x4_t*)(wrow[t] + k);
        ax[u][t] = *(const u32x4_t*)(xrow[t] + k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the step group issued first
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool step_ok = ks0 + u < nks;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x4_t av = (step_ok && mok[mt]) ? ax[u][mt] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = mfma16x16x32(as_bf16x8(av), as_bf16x8(bw[u][nt]), acc[mt][nt]);
      }
    }
  }
  float* dst = J.part + (int64_t)blockIdx.y * M * N + 64 * cb + (lane & 15);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mt + 4 * (lane >> 4) + r;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dst[(int64_t)m * N + 16 * nt] = acc[mt][nt][r];
    }
}

// Many-token (prefill) projection on MFMA: P[m][n] = sum_k x[m][k] W[n][k]
// with bf16 operands and float32 accumulation; x and W are both k-contiguous,
// so each operand row is read straight in the MFMA operand layout.  A
// work-group of 4 waves takes a 128 x 128 tile of P (each wave 64 x 64, 16
// accumulator tiles) and walks k in blocks of 64: a block's x and W tiles
// (16 KB each) are fetched into registers while the previous block is
// multiplied from LDS, then written to the other LDS buffer; one barrier per
// block.  LDS rows are padded to 72 bf16 so the 16-byte fragment reads of 16
// consecutive rows hit distinct banks.
constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGPitch = kGK + 8;
constexpr int kGThreads = 256;

__global__ void __launch_bounds__(kGThreads) proj_tile_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wkv,
                                                              const uint16_t* __restrict__ wg,
                                                              int64_t M, int K, int CD,
                                                              float* __restrict__ P) {
  __shared__ uint16_t As[2][kGM * kGPitch];
  __shared__ uint16_t Bs[2][kGN * kGPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int N = 2 * CD;
  const int64_t m0 = (int64_t)blockIdx.y * kGM;
  const int n0 = blockIdx.x * kGN;
  // loader mapping: piece i = tid + 256 u (u < 4) is row i / 8, 16-byte column i % 8
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
  int soff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + kGThreads * u;
    const int r = i >> 3, c = (i & 7) * 8;
    int64_t m = m0 + r;
    m = m < M ? m : M - 1;  // ragged last tile: repeat the last row, never stored
    asrc[u] = x + m * K + c;
    const int n = n0 + r;
    bsrc[u] = (n < CD ? wkv + (int64_t)n * K : wg + (int64_t)(n - CD) * K) + c;
    soff[u] = r * kGPitch + c;
  }
  u32x4_t ra[4], rb[4];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = *(const u32x4_t*)(asrc[u] + k0);
      rb[u] = *(const u32x4_t*)(bsrc[u] + k0);
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *(u32x4_t*)(&As[buf][soff[u]]) = ra[u];
      *(u32x4_t*)(&Bs[buf][soff[u]]) = rb[u];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = K / kGK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) gload((kb + 1) * kGK);
#pragma unroll
    for (int s = 0; s < kGK / 32; ++s) {
      u32x4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *(const u32x4_t*)(&As[buf][(wm * 64 + 16 * i + r16) * kGPitch + 32 * s + 8 * kq]);
        bf[i] = *(const u32x4_t*)(&Bs[buf][(wn * 64 + 16 * i + r16) * kGPitch + 32 * s + 8 * kq]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma16x16x32(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
    }
    if (kb + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
  // D layout: row 4 kq + r of the A tile, column r16 of the B tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 64 + 16 * i + 4 * kq + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) P[m * N + n0 + wn * 64 + 16 * j + r16] = acc[i][j][r];
    }
}

static bool use_tile_proj(const csa_compress_args* a) {
  return a->x_fmt == CSA_BF16 && a->w_fmt == CSA_BF16 && a->dim % kGK == 0 &&
         (2 * (a->ratio == 4 ? 2 : 1) * a->head_dim) % kGN == 0;
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
  // block cache: entries through a block table, state in slots of a pool
  PageMap ent_pages;          // table == nullptr: entries[b][i]
  const int32_t* state_slot;  // nullptr: state of sequence b is slot b
  int64_t state_slots;
};

// State slot of sequence b, or -1 when it lies outside the pool (the
// sequence is then skipped).
__device__ __forceinline__ int64_t state_seq(const CompArgs& a, int64_t b) {
  if (!a.state_slot) return b;
  const int32_t sl = a.state_slot[b];
  return (sl >= 0 && sl < a.state_slots) ? sl : -1;
}

// Row of entry i of sequence b, or nullptr when it is not written (beyond
// the capacity, or in an unallocated block of a block cache).
__device__ __forceinline__ uint8_t* entry_row(const CompArgs& a, int64_t b, int64_t i) {
  if (i < 0 || i >= a.entries_cap) return nullptr;
  if (!a.ent_pages.table) return a.entries + ((size_t)b * (size_t)a.entries_cap + (size_t)i) * a.entry_rb;
  const int64_t r = paged_row(a.ent_pages, b, i);
  return r < 0 ? nullptr : a.entries + (size_t)r * a.entry_rb;
}

// (v, s) of token p of sequence b (state slot sq) at state column col
// (0 <= col < CD), where the call starts at p0.  Tokens before p0 are read
// from the state as given.
__device__ __forceinline__ void token_vs(const CompArgs& a, int64_t b, int64_t sq, int64_t p0,
                                         int64_t p, int col, float& v, float& s) {
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
  const int64_t si = (sq * (int64_t)(a.coff * a.ratio) + slot) * a.CD + col;
  v = a.kv_state[si];
  s = a.score_state[si];
}

// ------------------------------------------------------------------ emit
// Pool block i of sequence b (state slot st) into y[0, d) (reads only);
// returns this thread's sum of squares.
__device__ float pool_block(const CompArgs& a, int64_t b, int64_t st, int64_t p0, int64_t i,
                            float* y) {
  const int tid = threadIdx.x;
  const int r = a.ratio;
  const int d = a.d;
  // pool each channel over its slots: loads of 8 slots are issued together and
  // folded into a running max / sum (online softmax over the slot axis)
  float sq = 0.f;
  const int nslots = a.coff * r;
  for (int c = tid; c < d; c += kThreads) {
    float m = -INFINITY, l = 0.f, acc = 0.f;
    for (int sl0 = 0; sl0 < nslots; sl0 += 8) {
      float vv[8], ss[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sl = sl0 + j;
        if (sl >= nslots) { vv[j] = 0.f; ss[j] = -INFINITY; continue; }
        int64_t p;
        int col;
        if (a.coff == 2) {
          p = sl < r ? (i - 1) * r + sl : i * r + (sl - r);
          col = sl < r ? c : d + c;
        } else {
          p = i * r + sl;
          col = c;
        }
        token_vs(a, b, st, p0, p, col, vv[j], ss[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ss[j] == -INFINITY) continue;
        const float mn = fmaxf(m, ss[j]);
        const float sc = expf(m - mn);  // 0 while m is -inf
        const float e = expf(ss[j] - mn);
        l = l * sc + e;
        acc = acc * sc + e * vv[j];
        m = mn;
      }
    }
    const float C = acc / l;
    y[c] = C;
    sq = fmaf(C, C, sq);
  }
  return sq;
}

// Norm weights and rotation factors at position i * r of this thread's
// channels (d <= 512 = kPer TT, for work-groups of TT threads).
template <int TT = kThreads>
struct NormRopeT {
  static constexpr int kPer = 512 / TT;
  float gw[kPer], gp[kPer], cs[kPer], sn[kPer];
};
using NormRope = NormRopeT<>;
template <int TT = kThreads>
__device__ __forceinline__ NormRopeT<TT> load_norm_rope(const CompArgs& a, int64_t i) {
  const int tid = threadIdx.x;
  const int d = a.d;
  int64_t rrow = i * a.ratio;
  rrow = rrow < 0 ? 0 : (rrow >= a.rope_rows ? a.rope_rows - 1 : rrow);
  NormRopeT<TT> f;
#pragma unroll
  for (int u = 0; u < NormRopeT<TT>::kPer; ++u) {
    const int c = tid + u * TT;
    f.gw[u] = f.gp[u] = f.cs[u] = 1.f;
    f.sn[u] = 0.f;
    if (c < d) {
      f.gw[u] = a.norm_w[c];
      if (c >= d - kRopeDims) {
        const int k = (c - (d - kRopeDims)) >> 1;
        f.gp[u] = a.norm_w[c ^ 1];
        f.cs[u] = a.rope_cos[rrow * 32 + k];
        f.sn[u] = a.rope_sin[rrow * 32 + k];
      }
    }
  }
  return f;
}

// RMSNorm -> RoPE at position i * r -> optional Hadamard -> storage rounding of
// the pooled block in y; writes entry i of sequence b.  z: LDS scratch of d
// floats; f: load_norm_rope(a, i), fetched early so that its latency overlaps
// earlier work.
template <int TT = kThreads>
__device__ void finish_block(const CompArgs& a, int64_t b, int64_t i, float* y, float* z,
                             float* red, float sq, const NormRopeT<TT>& f) {
  static_assert(TT == 256 || TT == 512, "4 or 8 waves");
  constexpr int kPer = NormRopeT<TT>::kPer;
  const int tid = threadIdx.x;
  const int d = a.d;
  const float (&gw)[kPer] = f.gw, (&gp)[kPer] = f.gp, (&cs)[kPer] = f.cs, (&sn)[kPer] = f.sn;
  sq = wave_sum(sq);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  float ss = (red[0] + red[1]) + (red[2] + red[3]);  // wave sums, pairwise in a fixed order
  if (TT == 512) ss = ss + ((red[4] + red[5]) + (red[6] + red[7]));
  const float ms = ss / (float)d;
  const float inv = 1.0f / sqrtf(ms + a.eps);
  // normalise, and rotate the last 64 dims at position i * r (pairs 2k, 2k+1)
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * TT;
    if (c >= d) continue;
    const float v = y[c] * inv * gw[u];
    float out = v;
    if (c >= d - kRopeDims) {
      const float vp = y[c ^ 1] * inv * gp[u];
      out = (c & 1) ? (vp * sn[u] + v * cs[u]) : (v * cs[u] - vp * sn[u]);
    }
    z[c] = out;
  }
  __syncthreads();
  // Sylvester Hadamard (butterflies a+b, a-b at strides 1..d/2), scaled by
  // d^-1/2; with d <= 128 all butterflies belong to wave 0
  if (a.rotate) {
    const bool one_wave = d <= 128;
    if (!one_wave || tid < 64) {
      for (int h = 1; h < d; h <<= 1) {
        for (int q = tid; q < d / 2; q += TT) {
          const int lo = (q / h) * 2 * h + (q % h);
          const float u = z[lo], v = z[lo + h];
          z[lo] = u + v;
          z[lo + h] = u - v;
        }
        if (one_wave) wave_lds_sync(); else __syncthreads();
      }
    }
    if (one_wave) __syncthreads();
    const float sc = 1.0f / sqrtf((float)d);
    for (int c = tid; c < d; c += TT) z[c] *= sc;
    __syncthreads();
  }
  uint8_t* row = entry_row(a, b, i);
  if (row == nullptr) return;
  if (a.entry_fmt == CSA_F32) {
    for (int c = tid; c < d; c += TT) ((float*)row)[c] = z[c];
  } else if (a.entry_fmt == CSA_BF16) {
    for (int c = tid; c < d; c += TT) ((uint16_t*)row)[c] = f32_to_bf16(z[c]);
  } else {
    for (int c0 = 0; c0 < d; c0 += TT) {  // uniform trip count: whole waves call
      const int c = c0 + tid;
      const bool live = c < d;
      store_elem(a.entry_fmt, live ? z[c] : 0.f, c, d, live, row);
    }
  }
}

__global__ void __launch_bounds__(kThreads) emit_kernel(CompArgs a) {
  __shared__ float y[512];
  __shared__ float z[512];
  __shared__ float red[4];
  const int64_t b = blockIdx.y;
  const int64_t p0 = a.start_pos[b];
  const int r = a.ratio;
  const int64_t i = p0 / r + blockIdx.x;              // candidate block
  if (p0 < 0 || (i + 1) * r - 1 >= p0 + a.T) return;  // not completed by this call
  const int64_t st = state_seq(a, b);
  if (st < 0) return;
  const float sq = pool_block(a, b, st, p0, i, y);
  finish_block(a, b, i, y, z, red, sq, load_norm_rope(a, i));
}

// ------------------------------------------------------------------ state
// New slot contents after the call, as the token-by-token decode state machine
// leaves them: the unfinished block's tokens in their current slots; if a
// block completed in this call, every other current slot (and, with overlap,
// every previous slot) holds the last completed block.  Slots whose token
// precedes the call keep their value, except the overlap shift, which copies
// current slots into previous ones -- done from values read before any write.
__device__ void state_column(const CompArgs& a, int64_t b, int col) {
  const int64_t p0 = a.start_pos[b];
  if (p0 < 0) return;
  const int64_t sq = state_seq(a, b);
  if (sq < 0) return;
  const int r = a.ratio;
  const int64_t p1 = p0 + a.T;
  const int64_t first_block = p0 / r, end_block = p1 / r;
  const int nslots = a.coff * r;
  const int64_t sbase = sq * (int64_t)nslots * a.CD + col;
  const int64_t unfinished0 = end_block * r > p0 ? end_block * r : p0;
  if (a.coff == 1) {
    // no slot moves: tokens of this call land in slot p mod r
    for (int64_t p = unfinished0; p < p1; ++p) {
      float v, sc;
      token_vs(a, b, sq, p0, p, col, v, sc);
      a.kv_state[sbase + (p % r) * a.CD] = v;
      a.score_state[sbase + (p % r) * a.CD] = sc;
    }
    if (end_block > first_block) {
      const int64_t done = end_block - 1;
      for (int q = (int)(p1 - end_block * r); q < r; ++q) {
        const int64_t p = done * r + q;
        if (p < p0) continue;  // already in its slot
        float v, sc;
        token_vs(a, b, sq, p0, p, col, v, sc);
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
    token_vs(a, b, sq, p0, p, col, nv[sl], ns[sl]);
    wr[sl] = true;
  }
  if (end_block > first_block) {
    const int64_t done = end_block - 1;
    for (int q = 0; q < r; ++q) {
      const int64_t p = done * r + q;
      token_vs(a, b, sq, p0, p, col, nv[q], ns[q]);
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

__global__ void __launch_bounds__(kThreads) state_kernel(CompArgs a) {
  const int col = blockIdx.x * kThreads + threadIdx.x;
  if (col < a.CD) state_column(a, blockIdx.y, col);
}

// Single-token calls, one work-group per sequence: add the projection's k
// slices for the new token (score gets its slot bias) and write its slot; if
// the token completes a block, pool the block (the new token's values from
// registers, the others from the state), shift the current slots into the
// previous ones (overlap) and finish the entry.
// Single-token emit with overlap (ratio 4, 8 slots).  Everything this thread
// needs -- the projection slices of the new token, all 4 slot-bias rows, the
// 8 slots of its channels, and the norm weights and rotation factors of the
// block the token belongs to -- is loaded in one round, so the load phase is
// one round of memory latency.
template <int TT>
__device__ void emit_t1_overlap(const CompArgs& a, int64_t b, int64_t st, int64_t p0, float* y,
                                float* z, float* red) {
  const int r = 4, d = a.d, CD = a.CD, tid = threadIdx.x;
  const int N = 2 * CD;
  const int64_t sb = st * (int64_t)(2 * r) * CD;
  const NormRopeT<TT> nr = load_norm_rope<TT>(a, p0 < 0 ? 0 : p0 / r);
  constexpr int kPer = NormRopeT<TT>::kPer;  // channels per thread (d <= 512 = kPer TT)
  float pv[kPer][2][kKSlices], ps[kPer][2][kKSlices];  // slices of v and score, halves 0/1
  float ap[kPer][2][4];                                 // slot bias rows 0..3
  float sv[kPer][8], ssc[kPer][8];                      // slots 0..7 at their pooled column
  float c4v[kPer][4], c4s[kPer][4];                     // slots 4..7 at column c (shift)
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * TT < d ? tid + u * TT : d - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* pp = a.P + b * (int64_t)N + c + h * d;
#pragma unroll
      for (int ks = 0; ks < kKSlices; ++ks) {
        pv[u][h][ks] = pp[(int64_t)ks * a.B * N];
        ps[u][h][ks] = pp[(int64_t)ks * a.B * N + CD];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ap[u][h][q] = a.ape[(int64_t)q * CD + c + h * d];
    }
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int64_t si = sb + (int64_t)sl * CD + c + (sl >= r ? d : 0);
      sv[u][sl] = a.kv_state[si];
      ssc[u][sl] = a.score_state[si];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c4v[u][q] = a.kv_state[sb + (int64_t)(r + q) * CD + c];
      c4s[u][q] = a.score_state[sb + (int64_t)(r + q) * CD + c];
    }
  }
  if (p0 < 0) return;
  const int q0 = (int)(p0 % r);
  const int ns = r + q0;  // the new token's slot
  const bool done = q0 == r - 1;
  float sq = 0.f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * TT;
    if (c >= d) continue;
    float nv[2], nsc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float vs = pv[u][h][0], ss = ps[u][h][0];
#pragma unroll
      for (int ks = 1; ks < kKSlices; ++ks) {
        vs += pv[u][h][ks];
        ss += ps[u][h][ks];
      }
      float apv = ap[u][h][0];
#pragma unroll
      for (int q = 1; q < 4; ++q) apv = q == q0 ? ap[u][h][q] : apv;
      nv[h] = vs;
      nsc[h] = ss + apv;
    }
    if (!done) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a.kv_state[sb + (int64_t)ns * CD + c + h * d] = nv[h];
        a.score_state[sb + (int64_t)ns * CD + c + h * d] = nsc[h];
      }
      continue;
    }
    // the block completes: slot 7 is the new token (column c + d pooled)
    sv[u][7] = nv[1];
    ssc[u][7] = nsc[1];
    c4v[u][3] = nv[0];
    c4s[u][3] = nsc[0];
    float m = -INFINITY, l = 0.f, acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (ssc[u][j] == -INFINITY) continue;
      const float mn = fmaxf(m, ssc[u][j]);
      const float scl = expf(m - mn);
      const float e = expf(ssc[u][j] - mn);
      l = l * scl + e;
      acc = acc * scl + e * sv[u][j];
      m = mn;
    }
    // shift: slots 0..3 <- slots 4..7 (both halves); slot 7 keeps the new token
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a.kv_state[sb + (int64_t)q * CD + c] = c4v[u][q];
      a.score_state[sb + (int64_t)q * CD + c] = c4s[u][q];
      a.kv_state[sb + (int64_t)q * CD + d + c] = sv[u][4 + q];
      a.score_state[sb + (int64_t)q * CD + d + c] = ssc[u][4 + q];
    }
    a.kv_state[sb + (int64_t)ns * CD + c] = nv[0];
    a.score_state[sb + (int64_t)ns * CD + c] = nsc[0];
    a.kv_state[sb + (int64_t)ns * CD + d + c] = nv[1];
    a.score_state[sb + (int64_t)ns * CD + d + c] = nsc[1];
    const float C = acc / l;
    y[c] = C;
    sq = fmaf(C, C, sq);
  }
  if (!done) return;
  finish_block<TT>(a, b, p0 / r, y, z, red, sq, nr);
}

struct CompJobs {
  CompArgs c[kMaxJobs];
};

template <int TT>
__global__ void __launch_bounds__(TT) emit_t1_kernel(CompJobs jobs) {
  __shared__ float y[512];
  __shared__ float z[512];
  __shared__ float red[TT / 64];
  const CompArgs& a = jobs.c[blockIdx.y];
  const int64_t b = blockIdx.x;
  const int64_t p0 = a.start_pos[b];
  const int r = a.ratio;
  const int d = a.d, tid = threadIdx.x;
  const int nslots = a.coff * r;
  const int N = 2 * a.CD;
  const int64_t st = state_seq(a, b);
  if (st < 0) return;
  const int64_t sb = st * (int64_t)nslots * a.CD;
  if (a.coff == 2) {  // ratio 4 with overlap: 8 slots
    emit_t1_overlap<TT>(a, b, st, p0, y, z, red);
    return;
  }
  if (p0 < 0) return;
  const int ns = (a.coff == 2 ? r : 0) + (int)(p0 % r);  // the new token's slot
  const bool done = (p0 + 1) % r == 0;
  const int64_t i = p0 / r;
  const float* apr = a.ape + (int64_t)(p0 % r) * a.CD;
  float sq = 0.f;
  for (int c = tid; c < d; c += TT) {
    // new token: columns c (and d + c with overlap) of v and of the score
    float nv[2], nsc[2];
    const int halves = a.coff;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= halves) break;
      const int col = c + h * d;
      const float* pp = a.P + b * (int64_t)N + col;
      float sv = pp[0], ss = pp[a.CD];
#pragma unroll
      for (int ks = 1; ks < kKSlices; ++ks) {
        sv += pp[(int64_t)ks * a.B * N];
        ss += pp[(int64_t)ks * a.B * N + a.CD];
      }
      nv[h] = sv;
      nsc[h] = ss + apr[col];
    }
    if (!done) {
      for (int h = 0; h < halves; ++h) {
        a.kv_state[sb + (int64_t)ns * a.CD + c + h * d] = nv[h];
        a.score_state[sb + (int64_t)ns * a.CD + c + h * d] = nsc[h];
      }
      continue;
    }
    // with overlap, the shift moves current slots r..2r-1 of columns c and
    // d + c into slots 0..r-1; this thread alone touches these columns
    float shv[4], shs[4];
    if (a.coff == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool nw = r + q == ns;
        shv[q] = nw ? nv[0] : a.kv_state[sb + (int64_t)(r + q) * a.CD + c];
        shs[q] = nw ? nsc[0] : a.score_state[sb + (int64_t)(r + q) * a.CD + c];
      }
    }
    float m = -INFINITY, l = 0.f, acc = 0.f;
    float cur_v[4], cur_s[4];
    for (int sl0 = 0; sl0 < nslots; sl0 += 8) {
      float vv[8], ss[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sl = sl0 + j;
        const int hh = (a.coff == 2 && sl >= r) ? 1 : 0;
        const int col = c + hh * d;
        const int64_t si = sb + (int64_t)sl * a.CD + col;
        if (sl == ns) {
          vv[j] = nv[hh];
          ss[j] = nsc[hh];
        } else {
          vv[j] = sl < nslots ? a.kv_state[si] : 0.f;
          ss[j] = sl < nslots ? a.score_state[si] : -INFINITY;
        }
      }
      if (a.coff == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) { cur_v[q] = vv[4 + q]; cur_s[q] = ss[4 + q]; }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ss[j] == -INFINITY) continue;
        const float mn = fmaxf(m, ss[j]);
        const float scl = expf(m - mn);
        const float e = expf(ss[j] - mn);
        l = l * scl + e;
        acc = acc * scl + e * vv[j];
        m = mn;
      }
    }
    if (a.coff == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a.kv_state[sb + (int64_t)q * a.CD + c] = shv[q];
        a.score_state[sb + (int64_t)q * a.CD + c] = shs[q];
        a.kv_state[sb + (int64_t)q * a.CD + d + c] = cur_v[q];
        a.score_state[sb + (int64_t)q * a.CD + d + c] = cur_s[q];
      }
      // the new token's own slot keeps its value (as the state machine does)
      a.kv_state[sb + (int64_t)ns * a.CD + c] = nv[0];
      a.score_state[sb + (int64_t)ns * a.CD + c] = nsc[0];
      a.kv_state[sb + (int64_t)ns * a.CD + d + c] = nv[1];
      a.score_state[sb + (int64_t)ns * a.CD + d + c] = nsc[1];
    } else {
      a.kv_state[sb + (int64_t)ns * a.CD + c] = nv[0];
      a.score_state[sb + (int64_t)ns * a.CD + c] = nsc[0];
    }
    const float C = acc / l;
    y[c] = C;
    sq = fmaf(C, C, sq);
  }
  if (!done) return;
  finish_block<TT>(a, b, i, y, z, red, sq, load_norm_rope<TT>(a, i));
}

// ---- single-token calls of the 128-token (no overlap) compressor
// Pass 1, work-group (sequence b, 64-channel slice): the new token's slot from
// the projection slices (score plus slot bias); if the token completes a
// block, 8 threads per channel pool 16 slots each -- all of their loads in
// flight together -- and the 8 partial softmax sums are merged in order.
// Writes the pooled channels and the slice's sum of squares.
constexpr int kPoolChannels = 64;
constexpr int kPoolGroups = 8;                  // slot groups: one wave each
constexpr int kPoolSlots = 128 / kPoolGroups;   // slots per thread
constexpr int kPoolThreads = 64 * kPoolGroups;

__global__ void __launch_bounds__(kPoolThreads) pool128_t1_kernel(CompJobs jobs, float* ybuf,
                                                                float* sqbuf) {
  __shared__ float pm[kPoolGroups][kPoolChannels], pl[kPoolGroups][kPoolChannels],
      pa[kPoolGroups][kPoolChannels];
  const CompArgs& a = jobs.c[0];
  const int64_t b = blockIdx.x;
  const int slice = blockIdx.y;
  const int64_t p0 = a.start_pos[b];
  const int64_t st = state_seq(a, b);
  if (p0 < 0 || st < 0) return;
  const int r = a.ratio;                    // 128, one slot per token
  const int ns = (int)(p0 % r);
  const bool done = ns == r - 1;
  const int tid = threadIdx.x;
  const int cl = tid & (kPoolChannels - 1), g = tid >> 6;
  const int c = slice * kPoolChannels + cl;
  const int N = 2 * a.CD;
  const int64_t sb = st * (int64_t)r * a.CD;
  const bool own = ns / kPoolSlots == g;     // this slot group holds the new token
  float nv = 0.f, nsc = 0.f;
  if (own) {
    const float* pp = a.P + b * (int64_t)N + c;
    nv = pp[0];
    nsc = pp[a.CD];
#pragma unroll
    for (int ks = 1; ks < kKSlices; ++ks) {
      nv += pp[(int64_t)ks * a.B * N];
      nsc += pp[(int64_t)ks * a.B * N + a.CD];
    }
    nsc += a.ape[(int64_t)ns * a.CD + c];
    a.kv_state[sb + (int64_t)ns * a.CD + c] = nv;
    a.score_state[sb + (int64_t)ns * a.CD + c] = nsc;
  }
  if (!done) return;
  float vv[kPoolSlots], ss[kPoolSlots];
#pragma unroll
  for (int j = 0; j < kPoolSlots; ++j) {
    const int sl = kPoolSlots * g + j;
    const int64_t si = sb + (int64_t)sl * a.CD + c;
    vv[j] = sl == ns ? nv : a.kv_state[si];
    ss[j] = sl == ns ? nsc : a.score_state[si];
  }
  float m = -INFINITY, l = 0.f, acc = 0.f;
#pragma unroll
  for (int j = 0; j < kPoolSlots; ++j) {
    if (ss[j] == -INFINITY) continue;
    const float mn = fmaxf(m, ss[j]);
    const float scl = expf(m - mn);
    const float e = expf(ss[j] - mn);
    l = l * scl + e;
    acc = acc * scl + e * vv[j];
    m = mn;
  }
  pm[g][cl] = m;
  pl[g][cl] = l;
  pa[g][cl] = acc;
  __syncthreads();
  if (g != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int q = 0; q < kPoolGroups; ++q) M = fmaxf(M, pm[q][cl]);
  float L = 0.f, A = 0.f;
#pragma unroll
  for (int q = 0; q < kPoolGroups; ++q) {
    if (pm[q][cl] == -INFINITY) continue;
    const float wq = expf(pm[q][cl] - M);
    L += pl[q][cl] * wq;
    A += pa[q][cl] * wq;
  }
  const float C = A / L;
  ybuf[b * (int64_t)a.d + c] = C;
  const float sq = wave_sum(C * C);  // wave 0 holds the slice's 64 channels
  if (tid == 0) sqbuf[b * (a.d / kPoolChannels) + slice] = sq;
}

// Pass 2, one work-group per sequence whose block completed: RMSNorm -> RoPE
// -> storage rounding of the pooled row (slice sums of squares added in order).
__global__ void __launch_bounds__(kEmitT1Threads) finish128_t1_kernel(CompJobs jobs,
                                                                  const float* ybuf,
                                                                  const float* sqbuf) {
  __shared__ float y[512];
  __shared__ float z[512];
  __shared__ float red[kEmitT1Threads / 64];
  const CompArgs& a = jobs.c[0];
  const int64_t b = blockIdx.x;
  const int64_t p0 = a.start_pos[b];
  if (p0 < 0 || (p0 + 1) % a.ratio != 0 || state_seq(a, b) < 0) return;
  const int tid = threadIdx.x;
  for (int c = tid; c < a.d; c += kEmitT1Threads) y[c] = ybuf[b * (int64_t)a.d + c];
  float sq = 0.f;
  if (tid == 0) {
    const int ns = a.d / kPoolChannels;
    for (int q = 0; q < ns; ++q) sq += sqbuf[b * ns + q];
  }
  __syncthreads();
  finish_block<kEmitT1Threads>(a, b, p0 / a.ratio, y, z, red, sq,
                               load_norm_rope<kEmitT1Threads>(a, p0 / a.ratio));
}

}  // namespace

// The MFMA projection serves bf16 calls with B*T <= 64 and dim % 256 == 0.
static bool use_mfma_proj(const csa_compress_args* a) {
  const int64_t M = (int64_t)a->B * a->T;
  return a->x_fmt == CSA_BF16 && a->w_fmt == CSA_BF16 && M <= kMfmaMaxM && a->dim % 256 == 0;
}

// Single-token calls with bf16 operands take the K-sliced projection and the
// single-token emit.
static bool use_t1_slices(const csa_compress_args* a) {
  return a->T == 1 && a->x_fmt == CSA_BF16 && a->w_fmt == CSA_BF16 && a->dim % 256 == 0 &&
         (int64_t)a->B <= kSliceMaxM;
}

size_t compress_ws_bytes(const csa_compress_args* a) {
  const int coff = a->ratio == 4 ? 2 : 1;
  const int CD = coff * a->head_dim;
  if (use_t1_slices(a)) {  // per-slice partial products
    size_t b = align_up((size_t)kKSlices * a->B * 2 * CD * sizeof(float), 256);
    if (a->ratio == 128)  // pooled rows and slice sums of squares
      b += align_up((size_t)a->B * a->head_dim * sizeof(float), 256) +
           align_up((size_t)a->B * (a->head_dim / 64) * sizeof(float), 256);
    return b;
  }
  return align_up((size_t)a->B * a->T * 2 * CD * sizeof(float), 256);
}

static CompArgs comp_args(const csa_compress_args* in, float* P) {
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
  a.P = P;
  a.ent_pages = PageMap{nullptr, 0, 0, 0};
  if (in->block_table) {
    int shift = 0;
    while ((1 << shift) < in->block_entries) ++shift;
    a.ent_pages = PageMap{in->block_table, in->max_blocks, in->pool_blocks, shift};
    a.entries_cap = in->max_blocks * (int64_t)in->block_entries;
  }
  a.state_slot = in->state_slot;
  a.state_slots = in->state_slots;
  return a;
}

// Single-token bf16 calls with a common batch run as one projection launch
// and one emit launch.
static bool fusable(const csa_compress_args* in, int n) {
  if (n < 1 || n > kMaxJobs) return false;
  for (int i = 0; i < n; ++i)
    if (!use_t1_slices(&in[i]) || in[i].B != in[0].B ||
        (n > 1 && in[i].ratio == 128))
      return false;
  return true;
}

static hipError_t launch_fused_t1(const csa_compress_args* in, int n, void* ws, hipStream_t s) {
  ProjJobs pj;
  CompJobs cj;
  char* p = (char*)ws;
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    const int CD = (in[i].ratio == 4 ? 2 : 1) * in[i].head_dim;
    pj.j[i] = ProjJob{(const uint16_t*)in[i].x, (const uint16_t*)in[i].w_kv,
                      (const uint16_t*)in[i].w_gate, in[i].dim, CD, blocks, (float*)p};
    cj.c[i] = comp_args(&in[i], (float*)p);
    blocks += 2 * CD / 16;
    p += compress_ws_bytes(&in[i]);
  }
  for (int i = n; i < kMaxJobs; ++i) {
    pj.j[i] = pj.j[0];
    cj.c[i] = cj.c[0];
  }
  pj.n = n;
  const int M = in[0].B;
  if (M > kSliceRows) {  // several row blocks: the 64-column form
    ProjJobs pw = pj;
    int wblocks = 0;
    for (int i = 0; i < n; ++i) {
      pw.j[i].blk0 = wblocks;
      wblocks += 2 * pj.j[i].CD / 64;
    }
    for (int i = n; i < kMaxJobs; ++i) pw.j[i] = pw.j[0];
    hipLaunchKernelGGL(proj_slice_wide_kernel,
                       dim3(wblocks, kKSlices, (M + kSliceRows - 1) / kSliceRows), dim3(64), 0, s,
                       pw, M);
  } else {
    const int mt = (M + 15) / 16;
    const dim3 grid(blocks, kKSlices);
    if (mt == 1) hipLaunchKernelGGL(proj_slice_kernel<1>, grid, dim3(64), 0, s, pj, M);
    else if (mt == 2) hipLaunchKernelGGL(proj_slice_kernel<2>, grid, dim3(64), 0, s, pj, M);
    else if (mt == 3) hipLaunchKernelGGL(proj_slice_kernel<3>, grid, dim3(64), 0, s, pj, M);
    else hipLaunchKernelGGL(proj_slice_kernel<4>, grid, dim3(64), 0, s, pj, M);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n == 1 && in[0].ratio == 128) {  // pooling over 128 slots: split by channels
    const int CD = in[0].head_dim;
    float* ybuf = (float*)((char*)ws + align_up((size_t)kKSlices * M * 2 * CD * sizeof(float), 256));
    float* sqbuf = (float*)((char*)ybuf + align_up((size_t)M * in[0].head_dim * sizeof(float), 256));
    hipLaunchKernelGGL(pool128_t1_kernel, dim3(M, in[0].head_dim / kPoolChannels), dim3(kPoolThreads),
                       0, s, cj, ybuf, sqbuf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(finish128_t1_kernel, dim3(M), dim3(kEmitT1Threads), 0, s, cj,
                       (const float*)ybuf, (const float*)sqbuf);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(emit_t1_kernel<kEmitT1Threads>, dim3(M, n), dim3(kEmitT1Threads), 0, s, cj);
  return hipGetLastError();
}

size_t compress_many_ws_bytes(const csa_compress_args* in, int n) {
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += compress_ws_bytes(&in[i]);
  return b;
}

hipError_t launch_compress_many(const csa_compress_args* in, int n, void* ws, hipStream_t s) {
  if (fusable(in, n)) return launch_fused_t1(in, n, ws, s);
  char* p = (char*)ws;
  for (int i = 0; i < n; ++i) {
    hipError_t e = launch_compress(&in[i], p, s);
    if (e != hipSuccess) return e;
    p += compress_ws_bytes(&in[i]);
  }
  return hipSuccess;
}

hipError_t launch_compress(const csa_compress_args* in, void* ws, hipStream_t s) {
  if (use_t1_slices(in)) return launch_fused_t1(in, 1, ws, s);
  CompArgs a = comp_args(in, (float*)ws);
  float* P = (float*)ws;
  const int64_t M = (int64_t)in->B * in->T;
  const int N = 2 * a.CD;
  if (use_mfma_proj(in)) {
    const int mt = (int)((M + 15) / 16);
    ProjOut po{P, 0, in->start_pos, in->ape, in->ratio, a.coff, in->kv_state, in->score_state};
    dim3 grid(N / 16);
    const uint16_t* xp = (const uint16_t*)in->x;
    const uint16_t* wk = (const uint16_t*)in->w_kv;
    const uint16_t* wgp = (const uint16_t*)in->w_gate;
    if (mt == 1) hipLaunchKernelGGL(proj_mfma_kernel<1>, grid, dim3(kProjThreads), 0, s, xp, wk, wgp, (int)M, in->dim, a.CD, po);
    else if (mt == 2) hipLaunchKernelGGL(proj_mfma_kernel<2>, grid, dim3(kProjThreads), 0, s, xp, wk, wgp, (int)M, in->dim, a.CD, po);
    else if (mt == 3) hipLaunchKernelGGL(proj_mfma_kernel<3>, grid, dim3(kProjThreads), 0, s, xp, wk, wgp, (int)M, in->dim, a.CD, po);
    else hipLaunchKernelGGL(proj_mfma_kernel<4>, grid, dim3(kProjThreads), 0, s, xp, wk, wgp, (int)M, in->dim, a.CD, po);
  } else if (use_tile_proj(in)) {
    const uint16_t* xp = (const uint16_t*)in->x;
    for (int64_t m0 = 0; m0 < M; m0 += (int64_t)65535 * kGM) {
      const int64_t mm = M - m0 < (int64_t)65535 * kGM ? M - m0 : (int64_t)65535 * kGM;
      hipLaunchKernelGGL(proj_tile_kernel, dim3(N / kGN, (unsigned)((mm + kGM - 1) / kGM)),
                         dim3(kGThreads), 0, s, xp + m0 * in->dim, (const uint16_t*)in->w_kv,
                         (const uint16_t*)in->w_gate, mm, in->dim, a.CD, P + m0 * N);
    }
  } else if (M <= kGemvMaxM) {
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
