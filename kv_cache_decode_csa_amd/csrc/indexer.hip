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

// RNE to bf16, kept as a float (NaN stays NaN)
__device__ __forceinline__ float round_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return x;
  return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

constexpr int kIdxThreads = 256;
// Work-groups per row: Nmax / 4096 .. Nmax / 512 keys' worth, the fewest that
// give about 512 work-groups for the launch (a per-key score does not depend
// on it).
constexpr int kMinKeysPerWg = 512;
constexpr int kMaxKeysPerWg = 4096;
constexpr int64_t kTargetWgs = 512;
// 16-key MFMA tiles per wave step: FP8 rows are small enough to keep four
// tiles (64 keys, 8.4 KB per wave) and their successors in flight.
template <int KFMT> constexpr bool packed_key() { return KFMT == CSA_FP8_MX32 || KFMT == CSA_FP4_MX32; }
template <int KFMT> constexpr int tiles_per_iter() { return packed_key<KFMT>() ? 4 : 2; }
template <int KFMT> constexpr int key_row_bytes() {
  return KFMT == CSA_FP8_MX32 ? 132 : (KFMT == CSA_FP4_MX32 ? 68 : 256);
}

// Keys are read with a permuted contraction order: lane (r16, kq) holds, for
// key r16 of its tile, the 32 contiguous dims [32 kq, 32 kq + 32) -- one FP8
// scale group -- and MFMA k-step s covers dims {32 kq + 8 s + j}.  The query
// fragments use the same order, so every dot product is unchanged while each
// lane issues one contiguous 32-byte (FP8) or 64-byte (bf16) read per key.
struct KeyRaw {
  uint32_t w[16];   // fp8: w[0..7] codes, w[8] scale byte; fp4: w[0..3] codes, w[8] scale
                    // byte; bf16: w[0..15]
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
  } else if (KFMT == CSA_FP4_MX32) {
    const uint32_t* p = (const uint32_t*)(kr + 16 * kq);  // rows of 68 B: dword aligned
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = p[i];
    r.w[8] = kr[64 + kq];
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
  } else if (KFMT == CSA_FP4_MX32) {
    // dword s holds the 8 codes of dims 32 kq + 8 s .. +8 (element 2j low
    // nibble of byte j); the hardware conversion applies the power-of-two
    // scale exactly
    const uint32_t sb = r.w[8] & 0xffu;
    const float sc = sb == 0xffu ? __uint_as_float(0x7fc00000u) : exp2i((int)sb - 127);
    const uint32_t x = r.w[s];
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 0);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 1);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 2);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, sc, 3);
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
  return (16 * tiles_per_iter<KFMT>() * key_row_bytes<KFMT>()) / 16;
}
template <int KFMT> constexpr int stage_slots() {
  return packed_key<KFMT>() ? (stage_pieces<KFMT>() + 63) / 64 * 64
                            : 16 * tiles_per_iter<KFMT>() * 17;
}
template <int KFMT> __device__ __forceinline__ int stage_slot(int piece) {
  if (packed_key<KFMT>()) return piece;
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
  } else if (KFMT == CSA_FP4_MX32) {
    const uint32_t* L = (const uint32_t*)st + r * 17;  // 68 B = 17 dwords per row
#pragma unroll
    for (int i = 0; i < 4; ++i) f.w[i] = L[4 * kq + i];
    f.w[8] = L[16] >> (8 * kq);
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

// Scoring of one query row (the same for every kernel below): the query
// fragments and head weights live in registers; score() takes the fragment
// data of one step's tiles (get(nt, f)), forms the 16 heads x 16 keys MFMA
// products of every head tile, applies ReLU and the head weights, adds up the
// heads and records the step's scores.
//
// QF4: the queries are MXFP4-MX32 rows too (68 B per head), and one
// block-scaled FP4 MFMA (16 x 16 x 128, E8M0 scales) forms a tile's products
// over all 128 dims: lane (r16, kq) hands it the 32 E2M1 codes of block kq of
// head or key r16 with that block's scale, which is exactly how both rows are
// stored, so nothing is decoded.  The products of two scaled E2M1 values are
// exact, as they are in the bf16 MFMA of the decoded values.
template <int HT, int KFMT, int TILES = tiles_per_iter<KFMT>(), bool QF4 = false>
struct Scorer {
  static constexpr int kTiles = TILES;
  static_assert(TILES == 2 || TILES == 4, "a step is two or four 16-key tiles");
  static_assert(!QF4 || KFMT == CSA_FP4_MX32, "FP4 queries go with FP4 keys");
  uint4 qa[HT][4];  // A operand: head 16 mt + r16, dims 32 kq + 8 s .. +8 (QF4: qa[mt][0]
                    // the codes of block kq, qa[mt][1].x its scale byte)
  float wv[HT][4];  // head weights in the D layout: head 16 mt + 4 kq + r
  int r16, kq;
  bool bf16s;       // scores rounded to bf16 (RNE) before they are stored and ranked

  __device__ __forceinline__ void load(const uint16_t* q_idx, const float* w_idx, int64_t row,
                                       int lane, int bf16_scores) {
    constexpr int Hi = HT * 16;
    r16 = lane & 15;
    kq = lane >> 4;
    bf16s = bf16_scores != 0;
    if (QF4) {
      constexpr int kQRow = key_row_bytes<CSA_FP4_MX32>();  // 68 B per head
      const uint8_t* qrow = (const uint8_t*)q_idx + row * (int64_t)Hi * kQRow;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const uint8_t* h = qrow + (16 * mt + r16) * kQRow;
        const uint32_t* c = (const uint32_t*)(h + 16 * kq);  // 68-B rows: dword aligned
        qa[mt][0] = make_uint4(c[0], c[1], c[2], c[3]);
        qa[mt][1].x = h[64 + kq];
      }
    } else {
      const uint16_t* qrow = q_idx + row * (int64_t)Hi * kIndexDim;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          qa[mt][s] = *(const uint4*)(qrow + (16 * mt + r16) * kIndexDim + 32 * kq + 8 * s);
    }
    const float* wrow = w_idx + row * (int64_t)Hi;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[mt][r] = wrow[16 * mt + 4 * kq + r];
  }

  // The HT head tiles are independent accumulation chains: they are issued
  // round-robin so consecutive MFMAs do not wait on each other.
  __device__ __forceinline__ void tile_mfma(const KeyRaw& f, f32x4_t (&acc)[HT]) const {
    if (QF4) {
      typedef int v8i_t __attribute__((ext_vector_type(8)));
      const v8i_t kb = {(int)f.w[0], (int)f.w[1], (int)f.w[2], (int)f.w[3], 0, 0, 0, 0};
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const uint4 c = qa[mt][0];
        const v8i_t qb = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        // formats 4 / 4: E2M1 operands; the scale operands' byte 0 is used
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qb, kb, z, 4, 4, 0, (int)qa[mt][1].x, 0, (int)f.w[8]);
      }
      return;
    }
    bf16x8_t kb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kb[s] = key_frag<KFMT>(f, s);
#pragma unroll
    for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(as_bf16x8(qa[mt][s]), kb[s], acc[mt]);
  }

  // Partial score of a lane: the sum over its 16 heads (4 per head tile),
  // formed over 2 ReLU(x) = x + |x| (exact, and an abs is free on the adder);
  // the total is halved at the end.  Scaling by two commutes with every
  // rounding, so the result equals the plain sum of w_h ReLU(x_h) in the same
  // order, while a max would need its input canonicalized first.
  __device__ __forceinline__ float tile_partial(const f32x4_t (&acc)[HT]) const {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p += wv[mt][r] * (acc[mt][r] + fabsf(acc[mt][r]));
    return p;
  }

  // All tiles of a step (keys k .. k + 16 kTiles).  The four lane rows (kq)
  // hold partials over different heads; row exchanges add them up so that row
  // j ends with the scores of tile j (with two tiles, rows 2 and 3 repeat rows
  // 0 and 1), and the step's scores below `end` are written and counted in one
  // pass (only if `live`).
  // PACKED: hist holds two 16-bit counters per word (bin b in word b / 2, half b % 2).
  template <bool PACKED = false, class Get>
  __device__ __forceinline__ void score(int64_t k, bool live, int64_t end, Get&& get, float* srow,
                                        uint32_t* hist) const {
    float p[kTiles];
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
      KeyRaw f;
      get(nt, f);
      f32x4_t acc[HT];
      tile_mfma(f, acc);
      p[nt] = tile_partial(acc);
    }
    float a, c;
    if (kTiles == 4) {
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
    const float sc = bf16s ? round_bf16(0.5f * (a + c)) : 0.5f * (a + c);
    const int64_t key = k + 16 * kq + r16;
    if (live && (kTiles == 4 || kq < kTiles) && key < end) {
      srow[key] = sc;
      const uint32_t bin = score_key(sc) >> 20;
      if (PACKED) atomicAdd(&hist[bin >> 1], 1u << ((bin & 1u) << 4));
      else atomicAdd(&hist[bin], 1u);
    }
  }
};

// Block cache (PG): as in the split kernel below, a wave step's keys are at
// most two 32-key halves, each contiguous in one block; the ids of step i + 2
// are read right after step i's key loads, and a half in an unallocated block
// is staged as zeros.  The partial step at the end looks its keys up one by one.
template <int HT, int KFMT, bool PG>
__global__ void __launch_bounds__(kIdxThreads) index_scores_mfma(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores,
    int32_t* __restrict__ n_vis_out, uint32_t* __restrict__ hist_g, int bf16_scores, PageMap pm) {
  constexpr int64_t kRowBytes = key_row_bytes<KFMT>();
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

  Scorer<HT, KFMT> sc;
  sc.load(q_idx, w_idx, row, lane, bf16_scores);
  const int r16 = sc.r16, kq = sc.kq;
  __syncthreads();

  const uint8_t* kbase = PG ? k_idx : k_idx + b * Nmax * kRowBytes;
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
  auto score_tiles = [&](int64_t k, const KeyRaw (&f)[kTilesPerIter]) __attribute__((always_inline)) {
    sc.score(k, true, end, [&](int nt, KeyRaw& g) { g = f[nt]; }, srow, hist);
  };

  int64_t n_full = end - k0 >= kKeysPerIter ? (end - k0 - kKeysPerIter) / stride + 1 : 0;
  constexpr int kHalf = 32 * (int)kRowBytes / 16;  // pieces of 32 keys
  static_assert(kStagePieces <= 2 * kHalf, "a wave step spans at most two 32-key halves");
  if (n_full > 0) {
    u32x4_t* st_lds = stage[wave];
    // block ids of step i's halves (lane 0: first, lane 1: second), read with
    // a lane-dependent address so that they are vector loads
    auto tload = [&](int64_t i) __attribute__((always_inline)) {
      if (!PG) return 0;
      const int64_t k = k0 + (i < n_full ? i : 0) * stride;
      int64_t l = (k + 32 * (lane & 1)) >> pm.shift;
      l = l < pm.max_blocks ? l : pm.max_blocks - 1;
      return pm.table[b * pm.max_blocks + l];
    };
    struct Step {
      U4Array<kStageLoads> v;
      int zero;
    };
    auto gload = [&](int64_t i, int tid) __attribute__((always_inline)) {
      const int64_t k = k0 + i * stride;
      const u32x4_t* src0 = (const u32x4_t*)(kbase + k * kRowBytes);
      const u32x4_t* src1 = src0;
      Step st;
      st.zero = 0;
      if (PG) {
        const int64_t mask = ((int64_t)1 << pm.shift) - 1;
        const int id0 = __builtin_amdgcn_readlane(tid, 0);
        const int id1 = __builtin_amdgcn_readlane(tid, 1);
        const bool ok0 = id0 >= 0 && id0 < pm.pool_blocks;
        const bool ok1 = id1 >= 0 && id1 < pm.pool_blocks;
        st.zero = (ok0 ? 0 : 1) | (ok1 ? 0 : 2);
        src0 = (const u32x4_t*)(k_idx + (ok0 ? ((((int64_t)id0) << pm.shift) + (k & mask)) * kRowBytes : 0));
        src1 = (const u32x4_t*)(k_idx + (ok1 ? ((((int64_t)id1) << pm.shift) + ((k + 32) & mask)) * kRowBytes : 0));
      }
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        int piece = lane + 64 * j;
        piece = piece < kStagePieces ? piece : kStagePieces - 1;
        if (PG) st.v.v[j] = piece < kHalf ? src0[piece] : src1[piece - kHalf];
        else st.v.v[j] = src0[piece];
      }
      return st;
    };
    auto stage_and_score = [&](int64_t i, const Step& v) __attribute__((always_inline)) {
      wave_lds_sync();  // earlier reads of the region are ordered before these writes
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        const int piece = lane + 64 * j;
        const bool z = PG && ((v.zero >> (piece < kHalf ? 0 : 1)) & 1);
        st_lds[stage_slot<KFMT>(piece)] = z ? u32x4_t{0u, 0u, 0u, 0u} : v.v.v[j];
      }
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
    // ids of step i + 2 are read right after step i's keys (ta: even steps,
    // tb: odd steps)
    int ta = tload(0), tb = tload(1);
    Step sa = gload(0, ta), sb;
    ta = tload(2);
    int64_t i = 0;
    for (; i + 2 < n_full; i += 2) {
      sb = gload(i + 1, tb);
      tb = tload(i + 3);
      stage_and_score(i, sa);
      sa = gload(i + 2, ta);
      ta = tload(i + 4);
      stage_and_score(i + 1, sb);
    }
    if (i + 1 < n_full) {
      sb = gload(i + 1, tb);
      stage_and_score(i, sa);
      stage_and_score(i + 1, sb);
    } else {
      stage_and_score(i, sa);
    }
  }
  const int64_t kt = k0 + n_full * stride;
  if (kt < end) {
    KeyRaw f[kTilesPerIter];
    bool zk[kTilesPerIter];
#pragma unroll
    for (int nt = 0; nt < kTilesPerIter; ++nt) {
      int64_t key = kt + 16 * nt + r16;
      key = key < end ? key : end - 1;
      zk[nt] = false;
      if (PG) {
        const int64_t pr = paged_row(pm, b, key);
        zk[nt] = pr < 0;
        key = pr < 0 ? 0 : pr;
      }
      load_key<KFMT>(kbase + key * kRowBytes, kq, f[nt]);
    }
    if (PG) {
#pragma unroll
      for (int nt = 0; nt < kTilesPerIter; ++nt)
        if (zk[nt])
#pragma unroll
          for (int w = 0; w < 16; ++w) f[nt].w[w] = 0u;
    }
    score_tiles(kt, f);
  }
  __syncthreads();
  uint32_t* g = hist_g + row * kHistBins;
  for (int i = t; i < kHistBins; i += kIdxThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// FP8 and FP4 keys, producer/consumer form.  A work-group of 12 waves takes
// steps of 256 FP8 or 512 FP4 keys (33,792 or 34,816 bytes): the G
// work-groups of a row split its visible steps into G contiguous ranges of
// ceil(steps / G) (a contiguous stream per work-group measured faster than
// interleaved steps).  Waves 8..11 only load: loader j copies its quarter of
// a step (16 B per lane, pieces clamped into the visible rows) straight from
// global memory into LDS with the gfx950 direct-to-LDS loads, kSplitBufs - 1
// steps ahead of the scorers, into a ring of kSplitBufs LDS buffers; no
// registers hold the data on the way.  Waves 0..7 only score: the two
// scorers of a quarter take one half of it each (32 FP8 or 64 FP4 keys), two
// scorers per SIMD so that one's MFMAs overlap the other's vector work.  One
// work-group barrier per step: before it each loader waits (vmcnt) for its
// own loads of the step about to be scored; after it the loaders refill the
// buffer the scorers have just finished with.  Every wave runs n_steps
// iterations; loads past the work-group's last step repeat the last step's
// keys (just read, so in L2).  A step has a fixed cost of about 0.9 us (the
// barrier and each scorer's chain of LDS reads, MFMAs and score stores) on
// top of its bytes, so FP4 steps hold twice the keys: with 256-key steps the
// FP4 scan ran at 3.3 TB/s, and taking away three quarters of its MFMAs or
// its whole E2M1 decode did not change that.
//
// Block cache (PG): the keys sit in a pool of blocks of at least 32 keys, so
// each 32-key run of a quarter is contiguous in one block.  The block ids of
// a step's runs are read by scalar loads (their own counter, so waiting for
// them never waits for key loads) issued kSplitBufs - 1 steps before the
// step's keys.  A run whose block is unallocated is read from the pool's
// first block and overwritten with zeros in LDS before the barrier.
constexpr int kSplitScorers = 8;  // scorer waves, half a quarter each
constexpr int kSplitThreads = 64 * (kSplitScorers + 4);
template <int KF> constexpr int split_step() { return KF == CSA_FP8_MX32 ? 256 : 512; }
constexpr int kSplitBufs = 3;     // LDS buffers in the ring (steps in flight + 1)
constexpr int64_t kSplitTargetWgs = 256;

// s_waitcnt with vmcnt <= n and the other counters unconstrained (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A work-group barrier that orders no memory by itself: the compiler may not
// move memory operations across it, and no wait for outstanding loads or
// stores is implied.  The caller waits for what the other side will read
// (the loaders: their loads into LDS, by vmcnt).
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int HT, int KFMT, bool PG, bool QF4 = false>
__global__ void __launch_bounds__(kSplitThreads) index_scores_split(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores,
    int32_t* __restrict__ n_vis_out, uint32_t* __restrict__ hist_g, int bf16_scores, PageMap pm) {
  static_assert(KFMT == CSA_FP8_MX32 || KFMT == CSA_FP4_MX32, "packed key rows");
  constexpr int64_t kRowBytes = key_row_bytes<KFMT>();
  constexpr int kStep = split_step<KFMT>();
  constexpr int kSub = kStep / 4;                      // keys per quarter (one loader)
  constexpr int kHalfKeys = kSub / 2;                  // keys per scorer
  constexpr int kTiles = kHalfKeys / 16;               // 16-key MFMA tiles per scorer
  constexpr int kPieces = kSub * (int)kRowBytes / 16;  // 528 (FP8) or 544 pieces of 16 B
  constexpr int kLoads = (kPieces + 63) / 64;          // 9 per lane, the last one partial
  constexpr int kLastLanes = kPieces - 64 * (kLoads - 1);
  constexpr int kRuns = kSub / 32;                     // 32-key runs per quarter
  constexpr int kRun = 32 * (int)kRowBytes / 16;       // pieces per run: 264 or 136
  static_assert(kSub * (int)kRowBytes % 16 == 0 && kRuns <= 4, "whole pieces, at most 4 runs");
  __shared__ uint32_t hist[kHistBins];
  __shared__ __attribute__((aligned(16))) u32x4_t buf[kSplitBufs][4][kPieces];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool loader = wave >= kSplitScorers;
  const int j = loader ? wave - kSplitScorers : wave >> 1;  // quarter of the step
  const int64_t row = row_off + blockIdx.y;
  const int64_t b = row / Q;
  int64_t nv = ((int64_t)pos[row] + 1) / ratio;
  nv = nv < 0 ? 0 : (nv > Nmax ? Nmax : nv);
  if (blockIdx.x == 0 && t == 0) n_vis_out[row] = (int32_t)nv;
  const int64_t G = gridDim.x;
  const int64_t row_steps = (nv + kStep - 1) / kStep;
  const int64_t per_wg = (row_steps + G - 1) / G;
  const int64_t s0 = (int64_t)blockIdx.x * per_wg;     // this work-group's first step
  if (s0 >= row_steps) return;
  const int64_t n_steps = row_steps - s0 < per_wg ? row_steps - s0 : per_wg;
  const uint8_t* kbase = PG ? k_idx : k_idx + b * Nmax * kRowBytes;
  const int64_t end = nv;

  for (int i = t; i < kHistBins; i += kSplitThreads) hist[i] = 0;
  __syncthreads();

  if (loader) {
    // the quarter's first key in step i; steps past the last repeat it
    auto step_key = [&](int64_t i) __attribute__((always_inline)) {
      const int64_t ii = s0 + (i < n_steps ? i : n_steps - 1);
      const int64_t k = ii * kStep + kSub * j;
      return k < end ? k : ii * kStep;
    };
    // block ids of step i's runs (uniform addresses: scalar loads)
    struct Ids { int id[kRuns]; };
    auto tload = [&](int64_t i) __attribute__((always_inline)) {
      Ids r;
#pragma unroll
      for (int u = 0; u < kRuns; ++u) r.id[u] = 0;
      if (!PG) return r;
      const int64_t k = step_key(i);
      // the table is read-only here: through the constant address space the
      // uniform loads become scalar loads
      typedef const __attribute__((address_space(4))) int32_t* ctab_t;
      const ctab_t tr = (ctab_t)(pm.table + b * pm.max_blocks);
#pragma unroll
      for (int u = 0; u < kRuns; ++u) {
        int64_t l = (k + 32 * u) >> pm.shift;
        l = l < pm.max_blocks ? l : pm.max_blocks - 1;
        r.id[u] = tr[l];
      }
      return r;
    };
    // issue step i's loads into LDS buffer `slot`; returns the zero bits
    // (bit u: run u's block is unallocated)
    auto issue = [&](int64_t i, int slot, const Ids& tid) __attribute__((always_inline)) {
      const int64_t k = step_key(i);
      const int64_t nk = end - k < kSub ? end - k : kSub;
      const int last = (int)((nk * kRowBytes - 1) / 16);
      const u32x4_t* src[kRuns];
      int zero = 0;
#pragma unroll
      for (int u = 0; u < kRuns; ++u) src[u] = (const u32x4_t*)(kbase + k * kRowBytes);
      if (PG) {
        const int64_t mask = ((int64_t)1 << pm.shift) - 1;
#pragma unroll
        for (int u = 0; u < kRuns; ++u) {
          const int id = tid.id[u];
          const bool ok = id >= 0 && id < pm.pool_blocks;
          zero |= ok ? 0 : 1 << u;
          src[u] = (const u32x4_t*)(k_idx + (ok ? ((((int64_t)id) << pm.shift) +
                                                   ((k + 32 * u) & mask)) * kRowBytes : 0)) -
                   kRun * u;
        }
      }
      u32x4_t* dst = buf[slot][j];
#pragma unroll
      for (int l = 0; l < kLoads; ++l) {
        const int piece = lane + 64 * l;
        const int p = piece < last ? piece : last;
        const u32x4_t* g = src[0] + p;
        if (PG) {
          const int run = p / kRun;
#pragma unroll
          for (int u = 1; u < kRuns; ++u) g = run == u ? src[u] + p : g;
        }
        if (l < kLoads - 1 || lane < kLastLanes)
          __builtin_amdgcn_global_load_lds((const void*)g,
                                           (__attribute__((address_space(3))) void*)(dst + 64 * l),
                                           16, 0, 0);
      }
      return zero;
    };
    // overwrite the unallocated runs of this quarter in buffer `slot`
    auto zero_runs = [&](int slot, int zero) __attribute__((always_inline)) {
      u32x4_t* dst = buf[slot][j];
      for (int piece = lane; piece < kPieces; piece += 64)
        if ((zero >> (piece / kRun)) & 1) dst[piece] = u32x4_t{0u, 0u, 0u, 0u};
    };
    // loads outstanding after a step's keys when the wait for that step is
    // issued: the later steps in flight
    constexpr int kAfter = (kSplitBufs - 2) * kLoads;
    // id pipeline (PG): tq[u] serves the steps issued at iterations
    // k = u mod (kSplitBufs - 1)
    constexpr int kT = kSplitBufs - 1;
    Ids tq[kT];
    int zr[kSplitBufs];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const Ids ids = tload(u);
      zr[u] = issue(u, u, ids);
      tq[u] = tload(u + kT);
    }
    zr[kSplitBufs - 1] = 0;
    int slot = 0;                      // buffer of step k
    auto body = [&](int64_t k, Ids& tqu) __attribute__((always_inline)) {
      wait_vmcnt<kAfter>();            // this wave's loads of step k are in LDS
      int zk = 0;
#pragma unroll
      for (int u = 0; u < kSplitBufs; ++u) zk = u == slot ? zr[u] : zk;
      if (PG && zk) {
        zero_runs(slot, zk);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the zeros are in LDS
      }
      barrier_no_fence();              // step k to the scorers; step k - 1's buffer is free
      const int fill = slot == 0 ? kSplitBufs - 1 : slot - 1;
      const int zn = issue(k + kT, fill, tqu);
#pragma unroll
      for (int u = 0; u < kSplitBufs; ++u) zr[u] = u == fill ? zn : zr[u];
      tqu = tload(k + 2 * kT);
      slot = slot + 1 == kSplitBufs ? 0 : slot + 1;
    };
    for (int64_t k = 0; k < n_steps; k += kT) {
#pragma unroll
      for (int u = 0; u < kT; ++u)
        if (k + u < n_steps) body(k + u, tq[u]);
    }
    wait_vmcnt<0>();                   // no load into LDS outlives the kernel
  } else {
    Scorer<HT, KFMT, kTiles, QF4> sc;
    sc.load(q_idx, w_idx, row, lane, bf16_scores);
    float* srow = scores + row * Nmax;
    const int h = wave & 1;            // half of the quarter
    int slot = 0;
    for (int64_t k = 0; k < n_steps; ++k) {
      barrier_no_fence();              // the loaders have waited for step k's loads
      const u32x4_t* st = buf[slot][j];
      sc.score((s0 + k) * kStep + kSub * j + kHalfKeys * h, true, end,
               [&](int nt, KeyRaw& f) {
                 stage_read<KFMT>(st, kHalfKeys * h + 16 * nt + sc.r16, sc.kq, f);
               },
               srow, hist);
      slot = slot + 1 == kSplitBufs ? 0 : slot + 1;
    }
  }
  __syncthreads();
  uint32_t* g = hist_g + row * kHistBins;
  for (int i = t; i < kHistBins; i += kSplitThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// Many queries per sequence (chunked prefill), bf16 keys: the work is a
// dense contraction, so each key is read once per tile of kQT consecutive
// queries instead of once per query.  A work-group of kQT waves takes the
// tile's queries (wave j scores query j, with the query fragments of the
// per-query kernels) over a range of at most kQKeysPerWg keys: all threads
// load a step of 96 keys (24 KB) into registers while the previous step is
// scored from LDS, then store it to the other LDS buffer; one barrier per
// step.  Per key the scoring is the same MFMA chain, epilogue and order as the
// per-query bf16 kernel, so the scores are bit-identical to it.  The top
// radix digit is counted in LDS with two 16-bit counters per word (a range
// holds fewer than 2^16 keys) and flushed to the row histograms at the end.
constexpr int kQT = 12;                // queries per work-group (3 waves per SIMD)
constexpr int kQThreads = 64 * kQT;
constexpr int kQStep = 96;             // keys per step
constexpr int kQKeysPerWg = 32768;     // keys per work-group at most (16-bit counters)
constexpr int kQStageSlots = kQStep * 17;  // rows of 16 pieces, padded to 17
constexpr int kQLoads = kQStep * 16 / kQThreads;  // 16-byte pieces per thread per step
static_assert(kQLoads * kQThreads == kQStep * 16 && kQStep % 32 == 0, "whole pieces, 32-key calls");

template <int HT>
__global__ void __launch_bounds__(kQThreads) index_scores_qtile(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q,
    int64_t Nmax, int keys_per_wg, int64_t tile_off, float* __restrict__ scores,
    int32_t* __restrict__ n_vis_out, uint32_t* __restrict__ hist_g, int bf16_scores) {
  constexpr int KFMT = CSA_BF16;
  constexpr int64_t kRowBytes = 256;
  static_assert(tiles_per_iter<KFMT>() == 2, "a step is two scorer calls of 32 keys");
  __shared__ uint32_t hist[kQT][kHistBins / 2];
  __shared__ u32x4_t buf[2][kQStageSlots];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int tiles_per_seq = (Q + kQT - 1) / kQT;
  const int64_t tile = tile_off + blockIdx.y;
  const int64_t b = tile / tiles_per_seq;
  const int q0 = (int)(tile % tiles_per_seq) * kQT;
  const int qq = q0 + wave;
  const bool has_q = qq < Q;
  const int64_t row = b * Q + (has_q ? qq : Q - 1);
  auto visible = [&](int64_t r) {
    int64_t nv = ((int64_t)pos[r] + 1) / ratio;
    return nv < 0 ? 0 : (nv > Nmax ? Nmax : nv);
  };
  const int64_t nv = has_q ? visible(row) : 0;
  if (blockIdx.x == 0 && lane == 0 && has_q) n_vis_out[row] = (int32_t)nv;
  // the tile's key range: [x0, x1) clipped to the largest visible count
  int64_t nv_max = 0;
  for (int j = 0; j < kQT && q0 + j < Q; ++j) {
    const int64_t v = visible(b * Q + q0 + j);
    nv_max = v > nv_max ? v : nv_max;
  }
  const int64_t x0 = (int64_t)blockIdx.x * keys_per_wg;
  if (x0 >= nv_max) return;
  const int64_t x1 = x0 + keys_per_wg < nv_max ? x0 + keys_per_wg : nv_max;
  const int64_t n_steps = (x1 - x0 + kQStep - 1) / kQStep;
  const int64_t end = nv < x1 ? nv : x1;  // this query's keys in the range

  for (int i = t; i < kQT * kHistBins / 2; i += kQThreads) (&hist[0][0])[i] = 0;

  Scorer<HT, KFMT> sc;
  if (has_q) sc.load(q_idx, w_idx, row, lane, bf16_scores);
  float* srow = scores + row * Nmax;
  const uint8_t* kbase = k_idx + b * Nmax * kRowBytes;
  // thread t loads pieces t + 512 u of a step: row p / 16, 16-byte column
  // p % 16, the row clamped into the range
  u32x4_t rg[kQLoads];
  auto gload = [&](int64_t i) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int p = t + kQThreads * u;
      int64_t key = x0 + i * kQStep + (p >> 4);
      key = key < x1 ? key : x1 - 1;
      rg[u] = ((const u32x4_t*)(kbase + key * kRowBytes))[p & 15];
    }
  };
  auto stage = [&](int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int p = t + kQThreads * u;
      buf[bi][(p >> 4) * 17 + (p & 15)] = rg[u];
    }
  };
  gload(0);
  stage(0);
  __syncthreads();
  for (int64_t i = 0; i < n_steps; ++i) {
    if (i + 1 < n_steps) gload(i + 1);
    if (has_q) {
      const u32x4_t* st = buf[i & 1];
      const int64_t k = x0 + i * kQStep;
#pragma unroll
      for (int h = 0; h < kQStep / 32; ++h)
        sc.template score<true>(k + 32 * h, true, end, [&](int nt, KeyRaw& f) {
          stage_read<KFMT>(st + 32 * h * 17, 16 * nt + sc.r16, sc.kq, f);
        }, srow, hist[wave]);
    }
    if (i + 1 < n_steps) stage((i + 1) & 1);
    __syncthreads();
  }
  // flush the nonzero counters of every query row of the tile
  for (int i = t; i < kQT * kHistBins / 2; i += kQThreads) {
    const int j = i / (kHistBins / 2), wd = i % (kHistBins / 2);
    if (q0 + j >= Q) continue;
    const uint32_t v = hist[j][wd];
    if (!v) continue;
    uint32_t* g = hist_g + (b * Q + q0 + j) * kHistBins + 2 * wd;
    if (v & 0xffffu) atomicAdd(&g[0], v & 0xffffu);
    if (v >> 16) atomicAdd(&g[1], v >> 16);
  }
}

// float32 path: one thread per key, q in LDS.
constexpr int kF32Keys = 256;
__global__ void __launch_bounds__(kIdxThreads) index_scores_f32(
    const float* __restrict__ q_idx, const float* __restrict__ w_idx,
    const float* __restrict__ k_idx, const int32_t* __restrict__ pos, int ratio, int Q, int Hi,
    int64_t Nmax, int64_t row_off, float* __restrict__ scores, int32_t* __restrict__ n_vis_out,
    uint32_t* __restrict__ hist_g, int bf16_scores, PageMap pm) {
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
    // a key in an unallocated block of a block cache reads as zeros
    const int64_t pr = pm.table ? paged_row(pm, b, key) : b * Nmax + key;
    const float* kr = k_idx + (pr < 0 ? 0 : pr) * kIndexDim;
    float kv[kIndexDim];
#pragma unroll
    for (int c = 0; c < kIndexDim; ++c) kv[c] = pr < 0 ? 0.f : kr[c];
    float p = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < kIndexDim; ++c) d = fmaf(qs[h * kIndexDim + c], kv[c], d);
      p = fmaf(ws[h], fmaxf(d, 0.f), p);
    }
    if (bf16_scores) p = round_bf16(p);
    scores[row * Nmax + key] = p;
    atomicAdd(&hist[score_key(p) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* g = hist_g + row * kHistBins;
  for (int i = t; i < kHistBins; i += kIdxThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

template <int HT, bool PG>
hipError_t launch_mfma_pg(const void* q_idx, int q_fmt, const float* w_idx, const void* k_idx, int k_fmt,
                          const int32_t* pos, int ratio, int Q, int64_t R, int64_t Nmax,
                          float* scores, int32_t* n_vis, uint32_t* hist, int bf16s, PageMap pm,
                          hipStream_t s) {
  if (!PG && k_fmt == CSA_BF16 && Q >= kQT) {
    // even ranges of at most kQKeysPerWg keys, whole steps
    const int64_t splits = (Nmax + kQKeysPerWg - 1) / kQKeysPerWg;
    int64_t kpw = (Nmax + splits - 1) / splits;
    kpw = (kpw + kQStep - 1) / kQStep * kQStep;
    const int64_t tiles = R / Q * ((Q + kQT - 1) / kQT);
    for (int64_t y0 = 0; y0 < tiles; y0 += 65535) {
      const int64_t ny = tiles - y0 < 65535 ? tiles - y0 : 65535;
      hipLaunchKernelGGL((index_scores_qtile<HT>), dim3((unsigned)splits, (unsigned)ny),
                         dim3(kQThreads), 0, s, (const uint16_t*)q_idx, w_idx,
                         (const uint8_t*)k_idx, pos, ratio, Q, Nmax, (int)kpw, y0, scores, n_vis,
                         hist, bf16s);
    }
    return hipGetLastError();
  }
  if (k_fmt == CSA_FP8_MX32 || k_fmt == CSA_FP4_MX32) {
    // about one work-group per CU in all, at least one step each
    int64_t gx = (kSplitTargetWgs + R - 1) / R;
    const int kStep = k_fmt == CSA_FP8_MX32 ? split_step<CSA_FP8_MX32>() : split_step<CSA_FP4_MX32>();
    const int64_t steps = (Nmax + kStep - 1) / kStep;
    gx = gx < steps ? gx : steps;
    gx = gx < 1 ? 1 : gx;
    for (int64_t r0 = 0; r0 < R; r0 += 65535) {
      int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)nr), dim3(kSplitThreads), 0, s,
                           (const uint16_t*)q_idx, w_idx, (const uint8_t*)k_idx, pos, ratio, Q,
                           Nmax, r0, scores, n_vis, hist, bf16s, pm);
      };
      if (k_fmt == CSA_FP8_MX32) go(index_scores_split<HT, CSA_FP8_MX32, PG>);
      else if (q_fmt == CSA_FP4_MX32) go(index_scores_split<HT, CSA_FP4_MX32, PG, true>);
      else go(index_scores_split<HT, CSA_FP4_MX32, PG>);
    }
    return hipGetLastError();
  }
  int kpw = kMaxKeysPerWg;
  while (kpw > kMinKeysPerWg && R * ((Nmax + kpw - 1) / kpw) < kTargetWgs) kpw >>= 1;
  const int64_t gx = (Nmax + kpw - 1) / kpw;
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    hipLaunchKernelGGL((index_scores_mfma<HT, CSA_BF16, PG>), dim3((unsigned)gx, (unsigned)nr),
                       dim3(kIdxThreads), 0, s, (const uint16_t*)q_idx, w_idx,
                       (const uint8_t*)k_idx, pos, ratio, Q, Nmax, r0, scores, n_vis, hist,
                       bf16s, pm);
  }
  return hipGetLastError();
}

template <int HT>
hipError_t launch_mfma(const void* q_idx, int q_fmt, const float* w_idx, const void* k_idx, int k_fmt,
                       const int32_t* pos, int ratio, int Q, int64_t R, int64_t Nmax,
                       float* scores, int32_t* n_vis, uint32_t* hist, int bf16s, PageMap pm,
                       hipStream_t s) {
  if (pm.table)
    return launch_mfma_pg<HT, true>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores,
                                    n_vis, hist, bf16s, pm, s);
  return launch_mfma_pg<HT, false>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores,
                                   n_vis, hist, bf16s, pm, s);
}

}  // namespace

hipError_t launch_index_scores(const void* q_idx, int q_fmt, const float* w_idx,
                               const void* k_idx, int k_fmt, const int32_t* pos, int ratio, int B,
                               int Q, int Hi, int64_t Nmax, float* scores, int32_t* n_vis,
                               TopkWs w, int bf16_scores, hipStream_t s, PageMap pm) {
  const int64_t R = (int64_t)B * Q;
  if (k_fmt == CSA_F32) {
    int64_t gx = (Nmax + kF32Keys - 1) / kF32Keys;
    for (int64_t r0 = 0; r0 < R; r0 += 65535) {
      int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
      hipLaunchKernelGGL(index_scores_f32, dim3((unsigned)gx, (unsigned)nr), dim3(kIdxThreads), 0,
                         s, (const float*)q_idx, w_idx, (const float*)k_idx, pos, ratio, Q, Hi,
                         Nmax, r0, scores, n_vis, w.hist, bf16_scores, pm);
    }
    return hipGetLastError();
  }
  switch (Hi / 16) {
    case 1: return launch_mfma<1>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 2: return launch_mfma<2>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 3: return launch_mfma<3>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 4: return launch_mfma<4>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 5: return launch_mfma<5>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 6: return launch_mfma<6>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 7: return launch_mfma<7>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    case 8: return launch_mfma<8>(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, Q, R, Nmax, scores, n_vis, w.hist, bf16_scores, pm, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
