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
// Work-groups per row: Nmax / 4096 .. Nmax / 512 keys' worth, the fewest that
// give about 512 work-groups for the launch (a per-key score does not depend
// on it).
constexpr int kMinKeysPerWg = 512;
constexpr int kMaxKeysPerWg = 4096;
constexpr int64_t kTargetWgs = 512;
// 16-key MFMA tiles per wave step: FP8 rows are small enough to keep four
// tiles (64 keys, 8.4 KB per wave) and their successors in flight.
template <int KFMT> constexpr int tiles_per_iter() { return KFMT == CSA_FP8_MX32 ? 4 : 2; }

// Keys are read with a permuted contraction order: lane (r16, kq) holds, for
// key r16 of its tile, the 32 contiguous dims [32 kq, 32 kq + 32) -- one FP8
// scale group -- and MFMA k-step s covers dims {32 kq + 8 s + j}.  The query
// fragments use the same order, so every dot product is unchanged while each
// lane issues one contiguous 32-byte (FP8) or 64-byte (bf16) read per key.
struct KeyRaw {
  uint32_t w[16];   // fp8: w[0..7] codes, w[8] scale byte; bf16: w[0..15]
};

// Loads are unconditional (callers clamp the key index into the visible range)
// so that the wait before a step's MFMAs only covers that step's loads and the
// following step's loads stay in flight.
template <int KFMT>
__device__ __forceinline__ void load_key(const uint8_t* kr, int kq, KeyRaw& r) {
  if (KFMT == CSA_FP8_MX32) {
    const uint32_t* p = (const uint32_t*)(kr + 32 * kq);  // rows of 132 B: dword aligned
#pragma unroll
    for (int i = 0; i < 8; ++i) r.w[i] = p[i];
    r.w[8] = kr[128 + kq];
  } else {
    const uint4* p = (const uint4*)(kr + 64 * kq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = p[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
}

// k-step s operand (8 bf16) from the raw lane data; FP8 codes are decoded by
// the hardware scaled conversion (exact: E4M3 x 2^e fits bf16).
template <int KFMT>
__device__ __forceinline__ bf16x8_t key_frag(const KeyRaw& r, int s) {
  if (KFMT == CSA_FP8_MX32) {
    const float sc = exp2i((int)(r.w[8] & 0xffu) - 127);
    const uint32_t lo = r.w[2 * s], hi = r.w[2 * s + 1];
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
    uint4 u = make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                         __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
    return as_bf16x8(u);
  } else {
    return as_bf16x8(make_uint4(r.w[4 * s], r.w[4 * s + 1], r.w[4 * s + 2], r.w[4 * s + 3]));
  }
}


// ---- LDS staging of one step's keys (one wave's region)
// FP8: the step's 64 rows of 132 B are stored as the contiguous byte stream
// (528 pieces of 16 B; the last load's spare lanes land in unused slots).
// bf16: each 256-B row holds exactly 16 pieces; rows are padded to 272 B so
// the lanes of a fragment read hit distinct banks.
template <int KFMT> constexpr int stage_pieces() {
  return (16 * tiles_per_iter<KFMT>() * (KFMT == CSA_FP8_MX32 ? 132 : 256)) / 16;
}
template <int KFMT> constexpr int stage_slots() {
  return KFMT == CSA_FP8_MX32 ? (stage_pieces<KFMT>() + 63) / 64 * 64
                              : 16 * tiles_per_iter<KFMT>() * 17;
}
template <int KFMT> __device__ __forceinline__ int stage_slot(int piece) {
  if (KFMT == CSA_FP8_MX32) return piece;
  const int p = piece < stage_pieces<KFMT>() ? piece : stage_pieces<KFMT>() - 1;
  return (p >> 4) * 17 + (p & 15);
}
// Fragment data of key `r` of the step for lane quarter kq, as load_key gives it.
template <int KFMT>
__device__ __forceinline__ void stage_read(const u32x4_t* st, int r, int kq, KeyRaw& f) {
  if (KFMT == CSA_FP8_MX32) {
    const uint32_t* L = (const uint32_t*)st + r * 33;  // 132 B = 33 dwords per row
#pragma unroll
    for (int i = 0; i < 8; ++i) f.w[i] = L[8 * kq + i];
    f.w[8] = L[32] >> (8 * kq);
  } else {
    const u32x4_t* L = st + r * 17 + 4 * kq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t v = L[i];
      f.w[4 * i] = v.x; f.w[4 * i + 1] = v.y; f.w[4 * i + 2] = v.z; f.w[4 * i + 3] = v.w;
    }
  }
}
template <int N> struct U4Array {
  u32x4_t v[N];
};

// Orders this wave's LDS accesses around a write of data that other lanes of
// the same wave read (LDS operations of one wave execute in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int HT, int KFMT>
__global__ void __launch_bounds__(kIdxThreads) index_scores_mfma(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores,
    int32_t* __restrict__ n_vis_out, uint32_t* __restrict__ hist_g) {
  constexpr int Hi = HT * 16;
  constexpr int64_t kRowBytes = KFMT == CSA_FP8_MX32 ? 132 : 256;
  constexpr int kTilesPerIter = tiles_per_iter<KFMT>();
  constexpr int kKeysPerIter = 16 * kTilesPerIter;
  constexpr int kStagePieces = stage_pieces<KFMT>();
  constexpr int kStageLoads = (kStagePieces + 63) / 64;
  __shared__ uint32_t hist[kHistBins];
  __shared__ u32x4_t stage[4][stage_slots<KFMT>()];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t row = row_off + blockIdx.y;  // b * Q + q
  const int64_t b = row / Q;
  int64_t nv = ((int64_t)pos[row] + 1) / ratio;
  nv = nv < 0 ? 0 : (nv > Nmax ? Nmax : nv);
  if (blockIdx.x == 0 && t == 0) n_vis_out[row] = (int32_t)nv;
  // The G = gridDim.x work-groups of a row sweep it together: step i of wave w
  // in work-group x covers keys [((i G + x) 4 + w) K, +K).
  const int64_t G = gridDim.x;
  if ((int64_t)blockIdx.x * 4 * kKeysPerIter >= nv) return;

  for (int i = t; i < kHistBins; i += kIdxThreads) hist[i] = 0;

  const int r16 = lane & 15;
  const int kq = lane >> 4;
  // query fragments (A operand): head 16 mt + r16, dims 32 kq + 8 s .. +8
  uint4 qa[HT][4];
  const uint16_t* qrow = q_idx + row * (int64_t)Hi * kIndexDim;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[mt][s] = *(const uint4*)(qrow + (16 * mt + r16) * kIndexDim + 32 * kq + 8 * s);
  // head weights in the D layout: head 16 mt + 4 kq + r
  float wv[HT][4];
  const float* wrow = w_idx + row * (int64_t)Hi;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wrow[16 * mt + 4 * kq + r];
  __syncthreads();

  const uint8_t* kbase = k_idx + b * Nmax * kRowBytes;
  float* srow = scores + row * Nmax;
  const int64_t end = nv;
  // A full step (all K keys below `end`) is read as one contiguous, coalesced
  // byte stream (lane l takes 16-byte pieces l, l + 64, ...), put in the
  // wave's own LDS region and read back in the MFMA operand layout.  Two
  // register sets alternate, so the next step's stream is in flight while the
  // current one is scored.  A partial step at the end of the row (if any) is
  // read key by key with the index clamped to end - 1.
  const int64_t stride = G * 4 * (int64_t)kKeysPerIter;
  const int64_t k0 = ((int64_t)blockIdx.x * 4 + wave) * kKeysPerIter;
  // Scoring is split in two so that the MFMAs of one tile can be issued
  // before the partial sums of the previous one: tile_mfma forms the 16 heads
  // x 16 keys products of every head tile, tile_partial applies ReLU and the
  // head weights over the lane's heads.
  auto tile_mfma = [&](const KeyRaw& f, f32x4_t (&acc)[HT]) __attribute__((always_inline)) {
    bf16x8_t kb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kb[s] = key_frag<KFMT>(f, s);
    // the HT head tiles are independent accumulation chains: issue them
    // round-robin so consecutive MFMAs do not wait on each other
#pragma unroll
    for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(as_bf16x8(qa[mt][s]), kb[s], acc[mt]);
  };
  // Partial score of a lane: the sum over its 16 heads (4 per head tile),
  // formed over 2 ReLU(x) = x + |x| (exact, and an abs is free on the adder);
  // the total is halved at the end.  Scaling by two commutes with every
  // rounding, so the result equals the plain sum of w_h ReLU(x_h) in the same
  // order, while a max would need its input canonicalized first.
  auto tile_partial = [&](const f32x4_t (&acc)[HT]) __attribute__((always_inline)) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p += wv[mt][r] * (acc[mt][r] + fabsf(acc[mt][r]));
    return p;
  };
  // All tiles of a step, the MFMAs of tile nt + 1 ahead of the partial sums
  // of tile nt.  The four lane rows (kq) hold partials over different heads;
  // row exchanges add them up so that row j ends with the scores of tile j
  // (with two tiles, rows 2 and 3 repeat rows 0 and 1), and the step's scores
  // are written and counted in one pass.
  auto score_tiles = [&](int64_t k, const KeyRaw (&f)[kTilesPerIter]) __attribute__((always_inline)) {
    f32x4_t acc[2][HT];
    float p[kTilesPerIter];
    tile_mfma(f[0], acc[0]);
#pragma unroll
    for (int nt = 0; nt < kTilesPerIter; ++nt) {
      if (nt + 1 < kTilesPerIter) tile_mfma(f[nt + 1], acc[(nt + 1) & 1]);
      p[nt] = tile_partial(acc[nt & 1]);
    }
    float a, c;
    if (kTilesPerIter == 4) {
      swap_rows16(p[0], p[1]);
      swap_rows16(p[2], p[3]);
      a = p[0] + p[1];
      c = p[2] + p[3];
    } else {
      swap_rows16(p[0], p[1]);
      a = p[0] + p[1];
      c = a;
    }
    swap_halves32(a, c);
    const float sc = 0.5f * (a + c);
    const int64_t key = k + 16 * kq + r16;
    if ((kTilesPerIter == 4 || kq < kTilesPerIter) && key < end) {
      srow[key] = sc;
      atomicAdd(&hist[score_key(sc) >> 20], 1u);
    }
  };

  int64_t n_full = end - k0 >= kKeysPerIter ? (end - k0 - kKeysPerIter) / stride + 1 : 0;
  if (n_full > 0) {
    u32x4_t* st_lds = stage[wave];
    auto gload = [&](int64_t i) __attribute__((always_inline)) {
      const u32x4_t* src = (const u32x4_t*)(kbase + (k0 + i * stride) * kRowBytes);
      U4Array<kStageLoads> v;
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        int piece = lane + 64 * j;
        piece = piece < kStagePieces ? piece : kStagePieces - 1;
        v.v[j] = src[piece];
      }
      return v;
    };
    auto stage_and_score = [&](int64_t i, const U4Array<kStageLoads>& v)
                               __attribute__((always_inline)) {
      wave_lds_sync();  // earlier reads of the region are ordered before these writes
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) st_lds[stage_slot<KFMT>(lane + 64 * j)] = v.v[j];
      wave_lds_sync();
      KeyRaw f[kTilesPerIter];
#pragma unroll
      for (int nt = 0; nt < kTilesPerIter; ++nt) stage_read<KFMT>(st_lds, 16 * nt + r16, kq, f[nt]);
      score_tiles(k0 + i * stride, f);
    };
    // The loop body has no conditional part, so at its head only the
    // current step's loads are pending in every path (a skipped half would
    // leave loads pending into the other set, and the wait that then guards
    // that set would stall every iteration); the last one or two steps are
    // peeled, and no step is read twice.
    U4Array<kStageLoads> sa = gload(0), sb;
    int64_t i = 0;
    for (; i + 2 < n_full; i += 2) {
      sb = gload(i + 1);
      stage_and_score(i, sa);
      sa = gload(i + 2);
      stage_and_score(i + 1, sb);
    }
    if (i + 1 < n_full) {
      sb = gload(i + 1);
      stage_and_score(i, sa);
      stage_and_score(i + 1, sb);
    } else {
      stage_and_score(i, sa);
    }
  }
  const int64_t kt = k0 + n_full * stride;
  if (kt < end) {
    KeyRaw f[kTilesPerIter];
#pragma unroll
    for (int nt = 0; nt < kTilesPerIter; ++nt) {
      int64_t key = kt + 16 * nt + r16;
      key = key < end ? key : end - 1;
      load_key<KFMT>(kbase + key * kRowBytes, kq, f[nt]);
    }
    score_tiles(kt, f);
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
  int kpw = kMaxKeysPerWg;
  while (kpw > kMinKeysPerWg && R * ((Nmax + kpw - 1) / kpw) < kTargetWgs) kpw >>= 1;
  const int64_t gx = (Nmax + kpw - 1) / kpw;
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
