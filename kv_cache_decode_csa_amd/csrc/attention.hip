// Shared-KV multi-query attention with a sink over [window ; compressed] rows
// ("DeepSeek-V4 deep dive" section 3.1: one 512-d entry is key and value for
// every head; section 3.3: RoPE on the last 64 dims of q, inverse rotation of
// the output by the query's position; section 3.4 Eq. 27: the sink joins the
// softmax denominator only; sections 5.3 / 6.1: the list is the 128 window
// rows followed by the top-k (CSA) or all completed (HCA) entries).
//
// MFMA kernel layout (one work-group = 4 waves, 16 heads, one chunk of rows):
//   * rows are processed in tiles of 32; wave w owns dims [128w, 128w+128);
//   * every wave loads its 128-dim slice of the tile's rows straight into the
//     MFMA A-operand layout and forms a partial q.c over its slice; the four
//     partials are summed through LDS in a fixed order, so every wave holds the
//     full logits and runs the same online softmax;
//   * for the value product the wave stores its slice row-major in LDS and
//     reads it back with the transposing 16-bit LDS read, which hands every
//     lane 4 rows of one dim; P (16 heads x 32 rows, bf16) times that slice
//     accumulates O for 16 heads x its 128 dims in 32 accumulators;
//   * the next tile's rows are fetched while the current one is computed;
//   * each chunk leaves (m, l, O) per head; a merge kernel combines the chunks
//     in a fixed order, adds the sink, normalises and undoes the RoPE.
// Row formats are decoded exactly to bf16 on load (E4M3 x 2^e and E2M1 x E4M3
// both fit bf16's 8-bit significand).
#include <type_traits>

#include "common.h"

namespace csa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kTile = 32;             // rows per tile
constexpr int kChunkCsa = 64;         // rows per work-group, top-k lists
// With many queries per sequence (chunked prefill) there are enough (query,
// head group) units to fill the chip without splitting a list: a work-group
// then takes 640 rows -- the whole window + top-512 list -- and finishes the
// output itself, with no partials to write and merge.  The choice depends on
// the number of queries per sequence only, never on the batch.
constexpr int kChunkCsaLong = 640;
constexpr int kLongChunkMinQ = 16;
constexpr int kChunkHca = 1024;       // rows per work-group, dense lists
constexpr float kLog2e = 1.4426950408889634f;

struct RowRef {
  const uint8_t* p;  // row start, or nullptr when the row is absent
  int fmt;
};

// Dense lists from a block cache: a work-group resolves its chunk's rows
// through the block table once, into LDS (dynamic shared memory, 4 bytes per
// row), so the row loads of the tile loop keep their usual depth.  Chunks of
// paged dense lists never exceed this (the launcher picks the kernel so).
constexpr int kPagedIdsMax = 2048;

// The window of sequence b: b itself, or its state slot (-1 when the slot
// lies outside the pool: the window rows are then absent).
__device__ __forceinline__ int64_t win_seq(const AttnArgs& a, int64_t b) {
  if (!a.win_slot) return b;
  const int32_t sl = a.win_slot[b];
  return (sl >= 0 && sl < a.win_slots) ? sl : -1;
}

// Row of list id e of entry set be: e itself in the contiguous layout, the
// pool row through the block table, or -1 when the id is absent.
__device__ __forceinline__ int32_t ent_row_id(const AttnArgs& a, int64_t be, int32_t e) {
  if (e < 0 || e >= a.Nmax) return -1;
  return a.ent_pages.table ? (int32_t)paged_row(a.ent_pages, be, e) : e;
}

// First row of entry set be (the pool itself through a block table).
__device__ __forceinline__ const uint8_t* ent_base(const AttnArgs& a, int64_t be) {
  return (const uint8_t*)a.entries +
         (a.ent_pages.table ? (size_t)0 : (size_t)be * (size_t)a.Nmax * a.ent_rb);
}

// Resolve logical list row j of unit (b, t); wsq is win_seq(a, b).
__device__ __forceinline__ RowRef resolve_row(const AttnArgs& a, int64_t unit, int64_t b,
                                              int64_t wsq, int t, int64_t j, int64_t nvis,
                                              size_t win_rb, size_t ent_rb) {
  RowRef r{nullptr, a.win_fmt};
  if (j < kWindow) {
    int64_t p = (int64_t)t - (kWindow - 1) + j;
    if (p < 0 || wsq < 0) return r;
    int64_t row;
    if (a.win_mode == CSA_WIN_RING128) {
      row = p & (kWindow - 1);
    } else {
      row = p - (int64_t)a.win_base[b];
      if (row < 0 || row >= a.win_rows) return r;
    }
    r.p = (const uint8_t*)a.win + ((size_t)wsq * (size_t)a.win_rows + (size_t)row) * win_rb;
    return r;
  }
  r.fmt = a.ent_fmt;
  const int64_t be = b % a.ent_seqs;
  int32_t e;
  if (a.dense) {
    if (j - kWindow >= nvis) return r;
    e = (int32_t)(j - kWindow);
  } else {
    if (j - kWindow >= a.topk) return r;
    e = a.topk_idx[(be * a.Q + (unit - b * a.Q)) * a.topk + (j - kWindow)];
  }
  e = ent_row_id(a, be, e);
  if (e < 0) return r;
  r.p = ent_base(a, be) + (size_t)e * ent_rb;
  return r;
}

__device__ __forceinline__ float row_val_f32(const RowRef& r, int d) {
  if (r.fmt == CSA_F32) return ((const float*)r.p)[d];
  if (r.fmt == CSA_BF16) return bf16_to_f32(((const uint16_t*)r.p)[d]);
  if (r.fmt == CSA_FP8_MX32)
    return e4m3_to_f32(r.p[d]) * exp2i((int)r.p[kHeadDim + (d >> 5)] - 127);
  uint32_t c = r.p[d >> 1];
  c = (d & 1) ? (c >> 4) : (c & 15u);
  return e2m1_to_f32(c) * e4m3_to_f32(r.p[kHeadDim / 2 + (d >> 4)]);
}

__device__ __forceinline__ int64_t unit_nvis(const AttnArgs& a, int t) {
  if (!a.dense) return 0;
  int64_t n = ((int64_t)t + 1) / a.ratio;
  return n < 0 ? 0 : (n > a.Nmax ? a.Nmax : n);
}

__device__ __forceinline__ int rope_row(const AttnArgs& a, int t) {
  int64_t r = t < 0 ? 0 : (int64_t)t;
  return (int)(r >= a.rope_rows ? a.rope_rows - 1 : r);
}

struct Partial {  // per (unit, head group, chunk)
  float m[16];
  float l[16];
  float o[16 * kHeadDim];
};

// Apply sink, normalise, inverse-RoPE and store one output value pair owner.
__device__ __forceinline__ void store_out(const AttnArgs& a, int64_t unit, int head, int d,
                                          float v) {
  int64_t i = (unit * a.H + head) * (int64_t)kHeadDim + d;
  if (a.out_fmt == CSA_F32) ((float*)a.out)[i] = v;
  else ((uint16_t*)a.out)[i] = f32_to_bf16(v);
}

// The chunks of a list are combined in chunk order by an online merge: a
// running maximum M and sum L per head (log2 units) and O rescaled at every
// step; a chunk with no visible row (mc = -inf) is skipped.  The merge kernel
// and the whole-list kernel both combine with these functions, in the same
// order, so they give the same bits.
// The running maximum after chunk mc, and the factors of the old sums (fa)
// and of the chunk's (fb).
// (The hardware exponential: both arguments are <= 0, and a factor below
// 2^-126 only scales terms that the factor-1 chunk outweighs.)
__device__ __forceinline__ float merge_factors(float M, float mc, float& fa, float& fb) {
  const float mn = fmaxf(M, mc);
  fa = __builtin_amdgcn_exp2f(M - mn);  // 0 while M is -inf
  fb = __builtin_amdgcn_exp2f(mc - mn);
  return mn;
}
// One sum (L, or an element of O) after folding in the chunk's value xc.
__device__ __forceinline__ float merge_o(float x, float xc, float fa, float fb) {
  return fmaf(xc, fb, x * fa);
}
// 1 / (L + 2^(sink - M)), the sink counted in the denominator only; 0 for a
// list with no visible row.
__device__ __forceinline__ float merge_inv(float M, float L, float sink2) {
  const float den = (M == -INFINITY) ? 0.f : L + exp2f(sink2 - M);
  return den > 0.f ? 1.f / den : 0.f;
}
// Inverse rotation of the pair (x, y) of dims (2k, 2k + 1) by the angle with
// cosine c and sine s.
__device__ __forceinline__ float unrot_even(float x, float y, float c, float s) {
  return fmaf(x, c, y * s);
}
__device__ __forceinline__ float unrot_odd(float x, float y, float c, float s) {
  return fmaf(y, c, -(x * s));
}

// ------------------------------------------------------------------ MFMA kernel
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Transposed 16-bit LDS read: inside each 16-lane group, lane j supplies the 4
// values at its address and lane c receives value c%4 of lane 4i + c/4 as its
// element i.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_t*)((__attribute__((address_space(3))) uint16_t*)p));
  return __builtin_bit_cast(uint2, v);
}

// Raw bytes of one row's 128-dim slice [128 w, 128 w + 128) as this lane
// needs them (dims 128 w + 32 s + 8 kq .. +8 for s = 0..3), per format.
template <int F> struct Raw;
template <> struct Raw<CSA_BF16> { uint4 v[4]; };
template <> struct Raw<CSA_FP8_MX32> { uint2 v[4]; uint32_t sc; };   // sc: groups 4w..4w+3
template <> struct Raw<CSA_FP4_E4M3_16> { uint32_t v[4]; uint2 sc; }; // sc: groups 8w..8w+7
// V4 mixed rows: FP8 codes of dims 0..447 (v[s]; scale bytes of blocks 2w,
// 2w+1 in sc) and, for wave 3, the bf16 dims 448..479 in v[2], v[3] and
// 480..511 in t
template <> struct Raw<CSA_MIX576> { uint2 v[4]; uint4 t; uint32_t sc; };

// Loads are unconditional: an absent row is read from a stand-in row of the
// same buffer and zeroed when its fragments are formed, so the wait before a
// tile's MFMAs covers only that tile's loads.
template <int F>
__device__ __forceinline__ void load_raw(const uint8_t* p, int w, int kq, Raw<F>& r) {
  if (F == CSA_BF16) {
    Raw<CSA_BF16>& q = (Raw<CSA_BF16>&)r;
#pragma unroll
    for (int s = 0; s < 4; ++s) q.v[s] = *(const uint4*)(p + 2 * (128 * w + 32 * s + 8 * kq));
  } else if (F == CSA_FP8_MX32) {
    Raw<CSA_FP8_MX32>& q = (Raw<CSA_FP8_MX32>&)r;
#pragma unroll
    for (int s = 0; s < 4; ++s) q.v[s] = *(const uint2*)(p + 128 * w + 32 * s + 8 * kq);
    q.sc = *(const uint32_t*)(p + kHeadDim + 4 * w);
  } else if (F == CSA_MIX576) {
    Raw<CSA_MIX576>& q = (Raw<CSA_MIX576>&)r;
    q.v[0] = *(const uint2*)(p + 128 * w + 8 * kq);
    q.v[1] = *(const uint2*)(p + 128 * w + 32 + 8 * kq);
    if (w < 3) {
      q.v[2] = *(const uint2*)(p + 128 * w + 64 + 8 * kq);
      q.v[3] = *(const uint2*)(p + 128 * w + 96 + 8 * kq);
      q.t = make_uint4(0u, 0u, 0u, 0u);
    } else {
      const uint4 a = *(const uint4*)(p + 448 + 16 * kq);
      q.v[2] = make_uint2(a.x, a.y);
      q.v[3] = make_uint2(a.z, a.w);
      q.t = *(const uint4*)(p + 512 + 16 * kq);
    }
    q.sc = (uint32_t)p[576 + 2 * w] | ((uint32_t)p[577 + 2 * w] << 8);
  } else {
    Raw<CSA_FP4_E4M3_16>& q = (Raw<CSA_FP4_E4M3_16>&)r;
#pragma unroll
    for (int s = 0; s < 4; ++s) q.v[s] = *(const uint32_t*)(p + 64 * w + 16 * s + 4 * kq);
    q.sc = *(const uint2*)(p + kHeadDim / 2 + 8 * w);
  }
}

// exact bf16 values of fragment s
template <int F>
__device__ __forceinline__ uint4 frag_bf16(const Raw<F>& r, int s, int kq) {
  if (F == CSA_BF16) {
    return ((const Raw<CSA_BF16>&)r).v[s];
  } else if (F == CSA_FP8_MX32) {
    const Raw<CSA_FP8_MX32>& q = (const Raw<CSA_FP8_MX32>&)r;
    const float sc = exp2i((int)((q.sc >> (8 * s)) & 0xffu) - 127);
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].x, sc, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].x, sc, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].y, sc, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].y, sc, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
  } else if (F == CSA_MIX576) {
    const Raw<CSA_MIX576>& q = (const Raw<CSA_MIX576>&)r;
    if ((threadIdx.x >> 6) == 3 && s >= 2)  // bf16 RoPE dims of wave 3
      return s == 2 ? make_uint4(q.v[2].x, q.v[2].y, q.v[3].x, q.v[3].y) : q.t;
    const float sc = exp2i((int)((q.sc >> (8 * (s >> 1))) & 0xffu) - 127);
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].x, sc, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].x, sc, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].y, sc, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.v[s].y, sc, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
  } else {
    const Raw<CSA_FP4_E4M3_16>& q = (const Raw<CSA_FP4_E4M3_16>&)r;
    const int g = 2 * s + (kq >> 1);  // group 8w + g
    const uint32_t sb = g < 4 ? (q.sc.x >> (8 * g)) : (q.sc.y >> (8 * (g - 4)));
    const float sc = e4m3_to_f32(sb & 0xffu);
    const uint32_t c = q.v[s];
    // byte j holds elements 2j (low nibble) and 2j + 1; the hardware
    // conversion (unit scale: it would apply only a power-of-two scale) gives
    // their exact E2M1 values, and the E4M3 scale is applied in float32 (the
    // product of a 2-bit and a 4-bit significand is exact, also in bf16)
    const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    return make_uint4(pack_bf16x2_exact(f0[0] * sc, f0[1] * sc),
                      pack_bf16x2_exact(f1[0] * sc, f1[1] * sc),
                      pack_bf16x2_exact(f2[0] * sc, f2[1] * sc),
                      pack_bf16x2_exact(f3[0] * sc, f3[1] * sc));
  }
}

constexpr int kRPitch = 128 + 16;  // bf16 per LDS row of a wave's 128-dim slice
// The 16-byte chunks of LDS row r are stored XOR-swizzled by bit 2 of r, so
// that both the fragment writes (8 rows per group of lanes) and the
// transposing reads (4 rows x 4 column pairs) hit distinct banks.
__device__ __forceinline__ int rswz(int row, int col) {  // bf16 offset of (row, col)
  return row * kRPitch + ((((col >> 3) ^ (row >> 2)) & 1) | ((col >> 3) & ~1)) * 8 + (col & 7);
}
constexpr int kMaxIdsPerLane = kChunkCsa / 16;

struct SoftmaxState {
  float m;      // running max (log2 units) of head r16
  float l;      // running denominator (without the sink)
  f32x4_t o[8]; // O for heads 4 kq + r, dims 128 w + 16 dt + r16
  int par;      // which of the two partial-logit buffers the next tile uses
};

// One 32-row tile: partial logits over this wave's dims, fixed-order sum of
// the 4 waves' partials through LDS, online softmax, O += P C.  One barrier
// per tile: R is this wave's own region (its earlier reads come first in
// program order), and consecutive tiles write alternate partial-logit
// buffers, so a wave that starts tile t + 1 cannot overwrite what a slower
// wave still reads of tile t (reaching tile t + 2 takes every wave past tile
// t + 1's barrier).
__device__ __forceinline__ void attend_tile(const uint4 (&fr)[2][4], uint32_t vmask,
                                            const uint4 (&qa)[4], float zscale, int w, int lane,
                                            uint16_t* R, float4 (*Spp)[4][2][64],
                                            SoftmaxState& st) {
  const int r16 = lane & 15, kq = lane >> 4;
  float4 (*Sp)[2][64] = Spp[st.par];
  st.par ^= 1;
  f32x4_t sacc[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    sacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sacc[rt] = mfma16x16x32(as_bf16x8(fr[rt][s]), as_bf16x8(qa[s]), sacc[rt]);
  }
  Sp[w][0][lane] = make_float4(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3]);
  Sp[w][1][lane] = make_float4(sacc[1][0], sacc[1][1], sacc[1][2], sacc[1][3]);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      *(uint4*)(R + rswz(16 * rt + r16, 32 * s + 8 * kq)) = fr[rt][s];
  __syncthreads();

  float z[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float4 acc = Sp[0][rt][lane];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      const float4 v = Sp[ww][rt][lane];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    z[rt][0] = acc.x; z[rt][1] = acc.y; z[rt][2] = acc.z; z[rt][3] = acc.w;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (vmask >> (16 * rt + 4 * kq + r)) & 1u;
      z[rt][r] = ok ? z[rt][r] * zscale : -INFINITY;
      tmax = fmaxf(tmax, z[rt][r]);
    }
  tmax = col_max4(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(st.m - m_new);
  float p[2][4];
  float psum = 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[rt][r] = (z[rt][r] == -INFINITY) ? 0.f : exp2f(z[rt][r] - m_new);
      psum += p[rt][r];
    }
  psum = col_sum4(psum);
  st.l = st.l * alpha + psum;
  st.m = m_new;
  // k index 8 kq + i <-> row 4 kq + i (i < 4) or 16 + 4 kq + i - 4, as in the logits
  float al[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * kq + r, 64);
  const bf16x8_t pa = as_bf16x8(make_uint4(pack_bf16x2(p[0][0], p[0][1]),
                                           pack_bf16x2(p[0][2], p[0][3]),
                                           pack_bf16x2(p[1][0], p[1][1]),
                                           pack_bf16x2(p[1][2], p[1][3])));
  const int rrow = 4 * kq + (r16 >> 2);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint2 c0 = lds_read_tr16(R + rswz(rrow, 16 * dt + 4 * (r16 & 3)));
    const uint2 c1 = lds_read_tr16(R + rswz(rrow + 16, 16 * dt + 4 * (r16 & 3)));
    f32x4_t acc = st.o[dt];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= al[r];
    st.o[dt] = mfma16x16x32(pa, as_bf16x8(make_uint4(c0.x, c0.y, c1.x, c1.y)), acc);
  }
}

// Rows [j0, j1) of the list, all in format F.  Two register sets alternate:
// while one tile is computed the next tile's rows are in flight.  Absent rows
// (and rows past j1) are loaded from `stand_in`, a row of the same buffer, and
// zeroed by the validity mask.  after_pair() runs after every two tiles, that
// is after rows [j0 + 64 i, j0 + 64 (i + 1)).
template <int F, class RowFn, class PairFn>
__device__ __forceinline__ void run_rows(int64_t j0, int64_t j1, RowFn row_of,
                                         const uint8_t* stand_in, const uint4 (&qa)[4],
                                         float zscale, int w, int lane, uint16_t* R,
                                         float4 (*Sp)[4][2][64], SoftmaxState& st,
                                         PairFn after_pair) {
  const int r16 = lane & 15, kq = lane >> 4;
  auto load_tile = [&](int64_t jt, Raw<F> (&f)[2], uint32_t& vm) {
    vm = 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t j = jt + 16 * rt + r16;
      const uint8_t* p = j < j1 ? row_of(j) : nullptr;
      const unsigned long long bal = __ballot(p != nullptr);
      vm |= (uint32_t)(bal & 0xffffull) << (16 * rt);
      load_raw<F>(p ? p : stand_in, w, kq, f[rt]);
    }
  };
  auto compute_tile = [&](const Raw<F> (&f)[2], uint32_t vm) {
    uint4 fr[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bool ok = (vm >> (16 * rt + r16)) & 1u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 v = frag_bf16<F>(f[rt], s, kq);
        fr[rt][s] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    attend_tile(fr, vm, qa, zscale, w, lane, R, Sp, st);
  };
  Raw<F> fa[2], fb[2];
  uint32_t va = 0, vb = 0;
  load_tile(j0, fa, va);
  for (int64_t jt = j0; jt < j1; jt += 2 * kTile) {
    load_tile(jt + kTile, fb, vb);
    compute_tile(fa, va);
    load_tile(jt + 2 * kTile, fa, va);
    if (jt + kTile < j1) compute_tile(fb, vb);
    after_pair();  // rows [jt, jt + 64) done
  }
}

// Pool rows of the dense chunk's entry rows [je, j_end) into ids[j - j_begin]
// (-1 where absent), by the whole work-group; ends with a barrier.
__device__ __forceinline__ void stage_paged_rows(const AttnArgs& a, int64_t be, int64_t j_begin,
                                                 int64_t je, int64_t j_end, int64_t nvis,
                                                 int32_t* ids) {
  for (int64_t j = je + threadIdx.x; j < j_end; j += kAttnThreads) {
    const int64_t e = j - kWindow;
    ids[j - j_begin] = e < nvis ? (int32_t)paged_row(a.ent_pages, be, e) : -1;
  }
  __syncthreads();
}

// Query slices for one wave: head tile ht of the work-group, dims
// 128 w + 32 s + 8 kq .. +8, with the last 64 dims rotated at row rr.  Every
// load (the fragments, and the rotation factors the wave needs) is issued
// before any is used.
template <int NH>
__device__ __forceinline__ void load_q_frags(const AttnArgs& a, int64_t unit, int head0, int w,
                                             int r16, int kq, int rr, uint4 (&qa)[NH][4]) {
#pragma unroll
  for (int ht = 0; ht < NH; ++ht) {
    const uint16_t* qp = (const uint16_t*)a.q + (unit * a.H + head0 + 16 * ht + r16) * (int64_t)kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[ht][s] = *(const uint4*)(qp + 128 * w + 32 * s + 8 * kq);
  }
  // dims >= 448 belong to wave 3, k-steps 2 and 3: pair k = 16 (s - 2) + 4 kq + j
  if (w != 3) return;
  float cs[2][4], sn[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[s][j] = a.rope_cos[(int64_t)rr * 32 + 16 * s + 4 * kq + j];
      sn[s][j] = a.rope_sin[(int64_t)rr * 32 + 16 * s + 4 * kq + j];
    }
#pragma unroll
  for (int ht = 0; ht < NH; ++ht)
#pragma unroll
    for (int s = 2; s < 4; ++s) {
      const uint4 raw = qa[ht][s];
      float v[8];
      const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(u[j] << 16);
        v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c = cs[s - 2][j], sv = sn[s - 2][j];
        const float x = v[2 * j], y = v[2 * j + 1];
        v[2 * j] = x * c - y * sv;
        v[2 * j + 1] = x * sv + y * c;
      }
      qa[ht][s] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
}

// ------------------------------------------------------------------ dense, all heads
// Dense lists (HCA) with H <= 64: one work-group serves every head, so each
// row is read once.  Waves still own 128 of the 512 dims; after the partial
// logits of all head tiles are summed through LDS, wave w runs the softmax of
// head tile w, and P and the rescale factors go through LDS so that every
// wave accumulates O for all heads over its dims.
// Rows per work-group: at least 512, and enough that a unit's list has at
// most kMergeChunks chunks, which the merge then combines in one round of
// loads (a multiple of the 32-row tile).
constexpr int kChunkDense = 512;
constexpr int kMergeChunks = 16;

template <int HT>
__device__ __forceinline__ void attend_tile_all(const uint4 (&fr)[2][4], uint32_t vmask,
                                                const uint4 (&qa)[HT][4], float zscale, int w,
                                                int lane, uint16_t* R, float4 (*Sp)[HT][2][64],
                                                uint4* Pl, float* Al, float& sm, float& sl,
                                                f32x4_t (&o)[HT][8]) {
  const int r16 = lane & 15, kq = lane >> 4;
  f32x4_t sacc[HT][2];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sacc[ht][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        sacc[ht][rt] = mfma16x16x32(as_bf16x8(fr[rt][s]), as_bf16x8(qa[ht][s]), sacc[ht][rt]);
  // No barrier before the writes: R is this wave's own region, the previous
  // tile's reads of Sp all come before its P barrier (which this wave has
  // passed), and Pl / Al are written only after the next barrier, which every
  // wave reaches after its previous P.C.
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      Sp[w][ht][rt][lane] = make_float4(sacc[ht][rt][0], sacc[ht][rt][1], sacc[ht][rt][2],
                                        sacc[ht][rt][3]);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      *(uint4*)(R + rswz(16 * rt + r16, 32 * s + 8 * kq)) = fr[rt][s];
  __syncthreads();
  if (w < HT) {  // softmax of head tile w
    float z[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float4 acc = Sp[0][w][rt][lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        const float4 v = Sp[ww][w][rt][lane];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      z[rt][0] = acc.x; z[rt][1] = acc.y; z[rt][2] = acc.z; z[rt][3] = acc.w;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vmask >> (16 * rt + 4 * kq + r)) & 1u;
        z[rt][r] = ok ? z[rt][r] * zscale : -INFINITY;
        tmax = fmaxf(tmax, z[rt][r]);
      }
    tmax = col_max4(tmax);
    const float m_new = fmaxf(sm, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(sm - m_new);
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[rt][r] = (z[rt][r] == -INFINITY) ? 0.f : exp2f(z[rt][r] - m_new);
        psum += p[rt][r];
      }
    psum = col_sum4(psum);
    sl = sl * alpha + psum;
    sm = m_new;
    Pl[w * 64 + lane] = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                   pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
    if (kq == 0) Al[16 * w + r16] = alpha;
  }
  __syncthreads();
  bf16x8_t pa[HT];
  float al[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    pa[ht] = as_bf16x8(Pl[ht * 64 + lane]);
#pragma unroll
    for (int r = 0; r < 4; ++r) al[ht][r] = Al[16 * ht + 4 * kq + r];
  }
  const int rrow = 4 * kq + (r16 >> 2);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint2 c0 = lds_read_tr16(R + rswz(rrow, 16 * dt + 4 * (r16 & 3)));
    const uint2 c1 = lds_read_tr16(R + rswz(rrow + 16, 16 * dt + 4 * (r16 & 3)));
    const bf16x8_t v = as_bf16x8(make_uint4(c0.x, c0.y, c1.x, c1.y));
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x4_t acc = o[ht][dt];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= al[ht][r];
      o[ht][dt] = mfma16x16x32(pa[ht], v, acc);
    }
  }
}

// Work-group = (chunk, unit, head part), chunk-major so that the short last
// chunks of the units run last.  A work-group takes HT head tiles; with
// hsplit > 1 the H / 16 head tiles are split over hsplit work-groups whose
// linear ids are 8 apart, so they run on one XCD at about the same time and
// read the chunk's rows through one L2 (work-groups are handed to the XCDs
// round-robin by linear id).  Writes one partial per (unit, head tile, chunk)
// in the layout of the merge kernel.
//
// SPARSE: a top-k list (CSA with many queries per sequence) in chunks of
// kChunkCsaLong rows, whose ids are staged in LDS.  A single-chunk list (the
// window + top-512) is finished here -- sink, normalisation, inverse RoPE,
// one rounding -- with no partials or merge.
template <int WF, int EF, int HT, bool SPARSE = false>
__global__ void __launch_bounds__(kAttnThreads, HT <= 2 ? 2 : 1) attn_dense_all_kernel(AttnArgs a, int chunk_rows,
                                                                      int nchunks, int64_t units,
                                                                      int hsplit, Partial* part) {
  __shared__ uint16_t Rl[4][kTile * kRPitch];
  __shared__ float4 Sp[4][HT][2][64];
  __shared__ uint4 Pl[HT * 64];
  __shared__ float Al[16 * HT];
  __shared__ int32_t Ids[SPARSE ? kChunkCsaLong : 1];

  int64_t item = blockIdx.x;
  int hs = 0;
  if (hsplit > 1) {
    const int64_t k = item >> 3;
    hs = (int)(k % hsplit);
    item = (k / hsplit) * 8 + (item & 7);
  }
  if (item >= (int64_t)nchunks * units) return;
  const int chunk = (int)(item / units);
  const int64_t unit = a.unit_off + item % units;
  const int ht0 = HT * hs;  // first head tile of this work-group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t b = unit / a.Q;
  // sequences share entry set (and top-k list) b % ent_seqs; sinks are [b / ent_seqs][H]
  const int64_t be = b % a.ent_seqs;
  const int64_t eunit = be * a.Q + (unit - b * a.Q);
  const float* sinks = a.sink + (b / a.ent_seqs) * a.H;
  const int t = a.pos[unit];
  const int64_t nvis = unit_nvis(a, t);
  const int64_t list_len = kWindow + (SPARSE ? (int64_t)a.topk : nvis);
  const int64_t j_begin = (int64_t)chunk * chunk_rows;
  int64_t j_end = j_begin + chunk_rows;
  if (j_end > list_len) j_end = list_len;
  const int rr = rope_row(a, t);
  const float zscale = a.scale * kLog2e;

  if (SPARSE) {  // the chunk's rows of the entry set (slot j - j_begin), -1 where absent
    for (int i = tid; i < kChunkCsaLong; i += kAttnThreads) {
      const int64_t jj = j_begin + i;
      Ids[i] = (jj >= kWindow && jj < j_end)
                   ? ent_row_id(a, be, a.topk_idx[eunit * a.topk + (jj - kWindow)])
                   : -1;
    }
    __syncthreads();
  }
  const int64_t wsq = win_seq(a, b);

  uint4 qa[HT][4];
  load_q_frags<HT>(a, unit, 16 * ht0, w, r16, kq, rr, qa);

  float sm = -INFINITY, sl = 0.f;
  f32x4_t o[HT][8];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* R = Rl[w];

  auto run = [&](auto fmt_tag, int64_t j0, int64_t j1, auto row_of, const uint8_t* stand_in) {
    constexpr int F = decltype(fmt_tag)::value;
    auto load_tile = [&](int64_t jt, Raw<F> (&f)[2], uint32_t& vm) {
      vm = 0;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int64_t j = jt + 16 * rt + r16;
        const uint8_t* p = j < j1 ? row_of(j) : nullptr;
        const unsigned long long bal = __ballot(p != nullptr);
        vm |= (uint32_t)(bal & 0xffffull) << (16 * rt);
        load_raw<F>(p ? p : stand_in, w, kq, f[rt]);
      }
    };
    auto compute_tile = [&](const Raw<F> (&f)[2], uint32_t vm) {
      uint4 fr[2][4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bool ok = (vm >> (16 * rt + r16)) & 1u;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 v = frag_bf16<F>(f[rt], s, kq);
          fr[rt][s] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      attend_tile_all<HT>(fr, vm, qa, zscale, w, lane, R, Sp, Pl, Al, sm, sl, o);
    };
    Raw<F> fa[2], fb[2];
    uint32_t va = 0, vb = 0;
    load_tile(j0, fa, va);
    for (int64_t jt = j0; jt < j1; jt += 2 * kTile) {
      load_tile(jt + kTile, fb, vb);
      compute_tile(fa, va);
      load_tile(jt + 2 * kTile, fa, va);
      if (jt + kTile < j1) compute_tile(fb, vb);
    }
  };

  // window rows [j_begin, min(j_end, 128))
  const int64_t jw = j_end < kWindow ? j_end : kWindow;
  if (j_begin < jw) {
    auto win_row = [&](int64_t j) -> const uint8_t* {
      return resolve_row(a, unit, b, wsq, t, j, nvis, a.win_rb, a.ent_rb).p;
    };
    const uint8_t* win0 =
        (const uint8_t*)a.win + (size_t)(wsq < 0 ? 0 : wsq) * (size_t)a.win_rows * a.win_rb;
    run(std::integral_constant<int, WF>{}, j_begin, jw, win_row, win0);
  }
  // entry rows [max(j_begin, 128), j_end)
  const int64_t je = j_begin > kWindow ? j_begin : kWindow;
  if (je < j_end && a.Nmax > 0) {
    const uint8_t* ebase = ent_base(a, be);
    // a dense list from a block cache: the chunk's pool rows, staged in LDS
    extern __shared__ int32_t PgIds[];
    const bool pg = !SPARSE && a.ent_pages.table != nullptr;
    if (pg) stage_paged_rows(a, be, j_begin, je, j_end, nvis, PgIds);
    auto ent_row = [&](int64_t j) -> const uint8_t* {
      if (SPARSE) {
        const int32_t e = Ids[j - j_begin];
        return e >= 0 ? ebase + (size_t)e * a.ent_rb : nullptr;
      }
      const int64_t e = j - kWindow;
      const int64_t r = pg ? (int64_t)PgIds[j - j_begin] : (e < nvis ? e : -1);
      return r >= 0 ? ebase + (size_t)r * a.ent_rb : nullptr;
    };
    run(std::integral_constant<int, EF>{}, je, j_end, ent_row, ebase);
  }

  if (SPARSE && nchunks == 1) {
    // finish: 1 / (l + e^{sink - m}) per head, shared through LDS (wave w holds
    // the softmax state of head tile w), then the inverse rotation of the
    // output's last 64 dims at the query's position and one rounding.  (Every
    // wave is past its last read of Al first.)
    __syncthreads();
    if (w < HT && kq == 0) {
      const float sink2 = sinks[16 * (ht0 + w) + r16] * kLog2e;
      const float den = (sm == -INFINITY) ? 0.f : sl + exp2f(sink2 - sm);
      Al[16 * w + r16] = den > 0.f ? 1.f / den : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float iv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) iv[r] = Al[16 * ht + 4 * kq + r];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = 128 * w + 16 * dt + r16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = o[ht][dt][r] * iv[r];
          const float nb = shfl_xor_f(v, 1);  // pair partner (d ^ 1)
          if (d >= kHeadDim - kRopeDims) {
            const int k = (d - (kHeadDim - kRopeDims)) >> 1;
            const float c = a.rope_cos[(int64_t)rr * 32 + k];
            const float sn = a.rope_sin[(int64_t)rr * 32 + k];
            v = (d & 1) ? (-nb * sn + v * c) : (v * c + nb * sn);
          }
          store_out(a, unit, 16 * (ht0 + ht) + 4 * kq + r, d, v);
        }
      }
    }
    return;
  }

  const int G = a.H / 16;
  if (w < HT && lane < 16) {
    Partial* P = part + (unit * G + ht0 + w) * (int64_t)nchunks + chunk;
    P->m[lane] = sm;
    P->l[lane] = sl;
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    Partial* P = part + (unit * G + ht0 + ht) * (int64_t)nchunks + chunk;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        P->o[(4 * kq + r) * kHeadDim + 128 * w + 16 * dt + r16] = o[ht][dt][r];
  }
}

// Work-group -> (chunk, unit, head group).  Work-groups are handed to the 8
// XCDs round-robin by linear id, so the head groups of one (chunk, unit) are
// given ids 8 apart: they run on the same XCD at about the same time and
// read the chunk's rows through one L2.
struct AttnItem {
  int chunk, hg;
  int64_t unit;
  bool live;
};

__device__ __forceinline__ AttnItem attn_item(const AttnArgs& a, int nchunks, int64_t units) {
  const int64_t L = blockIdx.x;
  const int G = a.H / 16;
  const int64_t k = L >> 3;
  const int64_t item = (k / G) * 8 + (L & 7);
  AttnItem it;
  it.hg = (int)(k % G);
  it.chunk = (int)(item % nchunks);
  it.unit = a.unit_off + item / nchunks;
  it.live = item < (int64_t)nchunks * units;
  return it;
}

// MODE kAttnChunks: chunks of kChunkCsa rows, ids held in registers, a
// partial per chunk.  MODE kAttnLong: chunks of kChunkCsaLong rows, whose
// top-k ids are staged in LDS.  MODE kAttnWhole: one work-group per list of
// at most kChunkCsaLong rows (ids in LDS) that runs the kChunkCsa-row chunks
// of kAttnChunks one after another, each with its own softmax state, and
// folds every chunk into a running merge as it ends, with the merge kernel's
// arithmetic and order: the output is bit for bit that of kAttnChunks and
// the merge, without partials in memory.
enum { kAttnChunks = 0, kAttnLong = 1, kAttnWhole = 2 };
template <int WF, int EF, int MODE>
__global__ void __launch_bounds__(kAttnThreads) attn_mfma_kernel(AttnArgs a, int chunk_rows,
                                                                 int nchunks, int64_t units,
                                                                 Partial* part) {
  constexpr bool LONG = MODE != kAttnChunks;  // ids staged in LDS
  constexpr bool WHOLE = MODE == kAttnWhole;
  static_assert(kChunkCsa == 2 * kTile, "a 64-row chunk is one pair of tiles of run_rows");
  static_assert(kWindow % kChunkCsa == 0, "chunks do not straddle the window and the entries");
  __shared__ uint16_t Rl[4][kTile * kRPitch];
  __shared__ float4 Sp[2][4][2][64];
  __shared__ int32_t Ids[LONG ? kChunkCsaLong : 1];

  const AttnItem it = attn_item(a, nchunks, units);
  if (!it.live) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t unit = it.unit;
  const int hg = it.hg;
  const int chunk = it.chunk;
  const int64_t b = unit / a.Q;
  // sequences share entry set (and top-k list) b % ent_seqs; sinks are [b / ent_seqs][H]
  const int64_t be = b % a.ent_seqs;
  const int64_t eunit = be * a.Q + (unit - b * a.Q);
  const float* sinks = a.sink + (b / a.ent_seqs) * a.H;
  const int t = a.pos[unit];
  const int64_t nvis = unit_nvis(a, t);
  const int64_t list_len = kWindow + (a.dense ? nvis : (int64_t)a.topk);
  const int64_t j_begin = (int64_t)chunk * chunk_rows;
  int64_t j_end = j_begin + chunk_rows;
  if (j_end > list_len) j_end = list_len;
  const int rr = rope_row(a, t);
  const float zscale = a.scale * kLog2e;

  // top-k ids of this chunk, fetched once: in registers (lane holds rows
  // j_begin + 16 i + r16), or for long chunks in LDS (slot j - j_begin);
  // both end up as rows of the entry set (pool rows through a block table),
  // -1 where absent
  int32_t ids[LONG ? 1 : kMaxIdsPerLane];
  if (!a.dense) {
    if (LONG) {
      for (int i = tid; i < kChunkCsaLong; i += kAttnThreads) {
        const int64_t jj = j_begin + i;
        Ids[i] = (jj >= kWindow && jj < j_end)
                     ? ent_row_id(a, be, a.topk_idx[eunit * a.topk + (jj - kWindow)])
                     : -1;
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int i = 0; i < kMaxIdsPerLane; ++i) {
        const int64_t jj = j_begin + 16 * i + r16;
        ids[i] = (jj >= kWindow && jj < j_end) ? a.topk_idx[eunit * a.topk + (jj - kWindow)] : -1;
      }
    }
  }

  // query slice: head 16 hg + r16, dims 128 w + 32 s + 8 kq .. +8, rotated
  uint4 qa1[1][4];
  load_q_frags<1>(a, unit, 16 * hg, w, r16, kq, rr, qa1);
  const uint4 qa[4] = {qa1[0][0], qa1[0][1], qa1[0][2], qa1[0][3]};
  // ids to rows after the query loads are issued, so that their round trips
  // overlap (a block table adds one more)
  if (!a.dense && !LONG) {
#pragma unroll
    for (int i = 0; i < kMaxIdsPerLane; ++i) ids[i] = ent_row_id(a, be, ids[i]);
  }
  const int64_t wsq = win_seq(a, b);

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.par = 0;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* R = Rl[w];

  // whole lists: the running merge of the chunks ended so far (head r16 for
  // M and L; O for heads 4 kq + r, dims 128 w + 16 dt + r16, as st.o)
  float Mw = -INFINITY, Lw = 0.f;
  f32x4_t ow[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ow[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto after_pair = [&]() {
    if (!WHOLE) return;
    float fa = 1.f, fb = 0.f;
    const int live = st.m != -INFINITY ? 1 : 0;
    if (live) {
      Mw = merge_factors(Mw, st.m, fa, fb);
      Lw = merge_o(Lw, st.l, fa, fb);
    }
    float ga[4], gb[4];
    int gl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ga[r] = __shfl(fa, 4 * kq + r, 64);
      gb[r] = __shfl(fb, 4 * kq + r, 64);
      gl[r] = __shfl(live, 4 * kq + r, 64);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (gl[r]) ow[dt][r] = merge_o(ow[dt][r], st.o[dt][r], ga[r], gb[r]);
      st.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    st.m = -INFINITY;
    st.l = 0.f;
  };

  // window rows [j_begin, min(j_end, 128))
  const int64_t jw = j_end < kWindow ? j_end : kWindow;
  if (j_begin < jw) {
    auto win_row = [&](int64_t j) -> const uint8_t* {
      return resolve_row(a, unit, b, wsq, t, j, nvis, a.win_rb, a.ent_rb).p;
    };
    const uint8_t* win0 =
        (const uint8_t*)a.win + (size_t)(wsq < 0 ? 0 : wsq) * (size_t)a.win_rows * a.win_rb;
    run_rows<WF>(j_begin, jw, win_row, win0, qa, zscale, w, lane, R, Sp, st, after_pair);
  }
  // entry rows [max(j_begin, 128), j_end)
  const int64_t je = j_begin > kWindow ? j_begin : kWindow;
  if (je < j_end && a.Nmax > 0) {
    const uint8_t* ebase = ent_base(a, be);
    if (a.dense) {
      // a dense list from a block cache: the chunk's pool rows, staged in LDS
      extern __shared__ int32_t PgIds[];
      const bool pg = a.ent_pages.table != nullptr;
      if (pg) stage_paged_rows(a, be, j_begin, je, j_end, nvis, PgIds);
      auto ent_row = [&](int64_t j) -> const uint8_t* {
        const int64_t e = j - kWindow;
        const int64_t r = pg ? (int64_t)PgIds[j - j_begin] : (e < nvis ? e : -1);
        return r >= 0 ? ebase + (size_t)r * a.ent_rb : nullptr;
      };
      run_rows<EF>(je, j_end, ent_row, ebase, qa, zscale, w, lane, R, Sp, st, after_pair);
    } else {
      auto ent_row = [&](int64_t j) -> const uint8_t* {
        int32_t e = -1;
        if (LONG) {
          e = Ids[j - j_begin];
        } else {
          // this lane's id slot for row j (rows are 16 r16-strided within the chunk)
          const int slot = (int)((j - j_begin) >> 4);
#pragma unroll
          for (int i = 0; i < kMaxIdsPerLane; ++i)
            if (i == slot) e = ids[i];
        }
        return e >= 0 ? ebase + (size_t)e * a.ent_rb : nullptr;
      };
      run_rows<EF>(je, j_end, ent_row, ebase, qa, zscale, w, lane, R, Sp, st, after_pair);
    }
  }

  // ---- chunk result
  if (WHOLE) {  // the merge kernel's finish on the running merge
    const float inv = merge_inv(Mw, Lw, sinks[16 * hg + r16] * kLog2e);
    float iv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) iv[r] = __shfl(inv, 4 * kq + r, 64);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 128 * w + 16 * dt + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = ow[dt][r] * iv[r];
        const float nb = shfl_xor_f(v, 1);  // pair partner (d ^ 1)
        if (d >= kHeadDim - kRopeDims) {
          const int k = (d - (kHeadDim - kRopeDims)) >> 1;
          const float c = a.rope_cos[(int64_t)rr * 32 + k];
          const float sn = a.rope_sin[(int64_t)rr * 32 + k];
          v = (d & 1) ? unrot_odd(nb, v, c, sn) : unrot_even(v, nb, c, sn);
        }
        store_out(a, unit, 16 * hg + 4 * kq + r, d, v);
      }
    }
    return;
  }
  if (nchunks > 1) {
    Partial* P = part + (unit * (a.H / 16) + hg) * (int64_t)nchunks + chunk;
    if (w == 0 && lane < 16) {
      P->m[lane] = st.m;
      P->l[lane] = st.l;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        P->o[(4 * kq + r) * kHeadDim + 128 * w + 16 * dt + r16] = st.o[dt][r];
    return;
  }
  // single chunk: finish here
  const float sink2 = sinks[16 * hg + r16] * kLog2e;
  const float den = (st.m == -INFINITY) ? 0.f : st.l + exp2f(sink2 - st.m);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float iv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) iv[r] = __shfl(inv, 4 * kq + r, 64);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int d = 128 * w + 16 * dt + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = st.o[dt][r] * iv[r];
      const float nb = shfl_xor_f(v, 1);  // pair partner (d ^ 1)
      if (d >= kHeadDim - kRopeDims) {
        const int k = (d - (kHeadDim - kRopeDims)) >> 1;
        const float c = a.rope_cos[(int64_t)rr * 32 + k];
        const float sn = a.rope_sin[(int64_t)rr * 32 + k];
        v = (d & 1) ? (-nb * sn + v * c) : (v * c + nb * sn);
      }
      store_out(a, unit, 16 * hg + 4 * kq + r, d, v);
    }
  }
}

// ------------------------------------------------------------------ merge
// One work-group per (unit, head group, 64-dim slice); thread t owns head t/16
// and 4 dims.  Chunks are folded in index order by the online merge; each
// batch of 16 chunks is loaded before any is folded, so the loads overlap.
constexpr int kMergeBatch = 16;
static_assert(kMergeChunks <= kMergeBatch, "a dense list merges in one round");

__global__ void __launch_bounds__(kAttnThreads, 4) attn_merge_kernel(AttnArgs a, int nchunks,
                                                                  const Partial* part) {
  const int tid = threadIdx.x;
  const int64_t unit = a.unit_off + blockIdx.y;
  const int G = a.H / 16;
  const int hg = blockIdx.x % G;
  const int slice = blockIdx.x / G;
  const Partial* P = part + (unit * G + hg) * (int64_t)nchunks;
  const int rr = rope_row(a, a.pos[unit]);
  const int h = tid >> 4;
  const int d0 = 64 * slice + 4 * (tid & 15);
  const float sink2 = a.sink[(unit / a.Q / a.ent_seqs) * a.H + 16 * hg + h] * kLog2e;
  float M = -INFINITY;
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nchunks; c0 += kMergeBatch) {
    // a batch of chunks loaded in one round, then folded in chunk order
    float mc[kMergeBatch], lc[kMergeBatch];
    float4 oc[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int c = c0 + i < nchunks ? c0 + i : nchunks - 1;
      mc[i] = P[c].m[h];
      lc[i] = P[c].l[h];
      oc[i] = *(const float4*)(P[c].o + h * kHeadDim + d0);
    }
    // the factors of every chunk first (the running maximum needs only the
    // chunk maxima, so the exponentials are independent), then the sums;
    // skipped chunks are dropped by selects, not branches
    bool live[kMergeBatch];
    float fa[kMergeBatch], fb[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      live[i] = c0 + i < nchunks && mc[i] != -INFINITY;
      const float mn = merge_factors(M, mc[i], fa[i], fb[i]);
      M = live[i] ? mn : M;
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      L = live[i] ? merge_o(L, lc[i], fa[i], fb[i]) : L;
      acc.x = live[i] ? merge_o(acc.x, oc[i].x, fa[i], fb[i]) : acc.x;
      acc.y = live[i] ? merge_o(acc.y, oc[i].y, fa[i], fb[i]) : acc.y;
      acc.z = live[i] ? merge_o(acc.z, oc[i].z, fa[i], fb[i]) : acc.z;
      acc.w = live[i] ? merge_o(acc.w, oc[i].w, fa[i], fb[i]) : acc.w;
    }
  }
  const float inv = merge_inv(M, L, sink2);
  float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (d0 >= kHeadDim - kRopeDims) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = (d0 - (kHeadDim - kRopeDims)) / 2 + j;
      const float c = a.rope_cos[(int64_t)rr * 32 + k];
      const float sn = a.rope_sin[(int64_t)rr * 32 + k];
      const float x = v[2 * j], y = v[2 * j + 1];
      v[2 * j] = unrot_even(x, y, c, sn);
      v[2 * j + 1] = unrot_odd(x, y, c, sn);
    }
  }
  const int64_t obase = (unit * a.H + 16 * hg + h) * (int64_t)kHeadDim + d0;
  if (a.out_fmt == CSA_F32)
    *(float4*)((float*)a.out + obase) = make_float4(v[0], v[1], v[2], v[3]);
  else
    *(uint2*)((uint16_t*)a.out + obase) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// ------------------------------------------------------------------ float32 kernel
// One work-group per (unit, head); thread t owns dims 2t and 2t+1.
__global__ void __launch_bounds__(kAttnThreads) attn_f32_kernel(AttnArgs a) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t unit = a.unit_off + blockIdx.y;
  const int head = blockIdx.x;
  const int64_t b = unit / a.Q;
  const float* sinks = a.sink + (b / a.ent_seqs) * a.H;  // sinks are [b / ent_seqs][H]
  const int t = a.pos[unit];
  const int rr = rope_row(a, t);
  const int64_t nvis = unit_nvis(a, t);
  const int64_t list_len = kWindow + (a.dense ? nvis : (int64_t)a.topk);
  const size_t win_rb = a.win_rb;
  const size_t ent_rb = a.ent_rb;
  const int d = 2 * tid;
  const float* qp = (const float*)a.q + (unit * a.H + head) * (int64_t)kHeadDim;
  float qx = qp[d], qy = qp[d + 1];
  const bool rot = d >= kHeadDim - kRopeDims;
  float rc = 1.f, rs = 0.f;
  if (rot) {
    const int k = (d - (kHeadDim - kRopeDims)) >> 1;
    rc = a.rope_cos[(int64_t)rr * 32 + k];
    rs = a.rope_sin[(int64_t)rr * 32 + k];
    const float nx = qx * rc - qy * rs, ny = qx * rs + qy * rc;
    qx = nx;
    qy = ny;
  }
  float m = -INFINITY, l = 0.f, ox = 0.f, oy = 0.f;
  const int64_t wsq = win_seq(a, b);
  for (int64_t j = 0; j < list_len; ++j) {
    RowRef rf = resolve_row(a, unit, b, wsq, t, j, nvis, win_rb, ent_rb);
    if (rf.p == nullptr) continue;  // uniform across the block
    const float cx = row_val_f32(rf, d), cy = row_val_f32(rf, d + 1);
    float part = fmaf(qx, cx, qy * cy);
    part = wave_sum(part);
    __syncthreads();
    if (lane == 0) red[w] = part;
    __syncthreads();
    const float z = ((red[0] + red[1]) + (red[2] + red[3])) * a.scale;
    const float mn = fmaxf(m, z);
    const float al = expf(m - mn);
    const float pz = expf(z - mn);
    l = l * al + pz;
    ox = ox * al + pz * cx;
    oy = oy * al + pz * cy;
    m = mn;
  }
  const float sink = sinks[head];
  const float den = (m == -INFINITY) ? 0.f : l + expf(sink - m);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float x = ox * inv, y = oy * inv;
  if (rot) {
    const float nx = x * rc + y * rs, ny = -x * rs + y * rc;
    x = nx;
    y = ny;
  }
  store_out(a, unit, head, d, x);
  store_out(a, unit, head, d + 1, y);
}

}  // namespace

static bool attn_long_chunks(const AttnArgs& a) {
  return !a.dense && a.Q >= kLongChunkMinQ && a.q_fmt != CSA_F32;
}

// Dense lists with at most 64 heads use the all-heads kernel (and always its
// merge); so do top-k lists with 64 heads and many queries per sequence
// (long chunks; a single-chunk list needs no merge).  Other lists use the
// 16-head-group kernel.
// Two work-groups of two head tiles each per item (ids 8 apart: one XCD, one
// L2 read of the rows): half the registers of one all-heads work-group, so two
// fit per SIMD; measured faster than one work-group of four head tiles.
constexpr int kSparseHsplit = 2;
static bool attn_sparse_all_heads(const AttnArgs& a) {
  return attn_long_chunks(a) && a.H == 64;
}
int64_t attn_list_len(const AttnArgs& a) {
  return kWindow + (a.dense ? a.Nmax : (int64_t)a.topk);
}

// Rows per chunk of a dense list in the all-heads kernel: at least
// kChunkDense, at most kMergeChunks chunks per list.
static int64_t dense_all_chunk_rows(const AttnArgs& a) {
  const int64_t per = (attn_list_len(a) + kMergeChunks - 1) / kMergeChunks;
  const int64_t cr = (per + kTile - 1) / kTile * kTile;
  return cr > kChunkDense ? cr : kChunkDense;
}

// A paged dense list takes the all-heads kernel only while its chunks fit
// the LDS row staging; longer ones take the head-group kernel's 1024-row chunks.
static bool attn_all_heads(const AttnArgs& a) {
  if (a.dense && a.H <= 64 && a.q_fmt != CSA_F32)
    return !a.ent_pages.table || dense_all_chunk_rows(a) <= kPagedIdsMax;
  return attn_sparse_all_heads(a);
}

// Top-k lists of at most kChunkCsaLong rows take one work-group per list
// (kAttnWhole) once the batch gives at least one (unit, head group) item per
// CU; smaller batches split each list over work-groups of kChunkCsa rows and
// merge the partials.  Both fold the same 64-row chunks in the same order with
// the same arithmetic, so the output does not depend on which runs, or on the
// batch.  Measured at top-512, FP8 rows, 64 heads: 56 against 65 us at 64
// sequences, 76 against 125 us at 128; at 48 sequences 54 against 52 us.
constexpr int64_t kWholeMinItems = 256;
static bool attn_whole_lists(const AttnArgs& a) {
  return !a.dense && a.q_fmt != CSA_F32 && !attn_long_chunks(a) &&
         attn_list_len(a) <= kChunkCsaLong &&
         (int64_t)a.B * a.Q * (a.H / 16) >= kWholeMinItems;
}

int attn_chunk_rows(const AttnArgs& a) {
  if (attn_long_chunks(a) || attn_whole_lists(a)) return kChunkCsaLong;
  if (!attn_all_heads(a)) return a.dense ? kChunkHca : kChunkCsa;
  return (int)dense_all_chunk_rows(a);
}

static int attn_nchunks(const AttnArgs& a) {
  int64_t L = attn_list_len(a);
  int cr = attn_chunk_rows(a);
  return (int)((L + cr - 1) / cr);
}

size_t attn_ws_bytes(const AttnArgs& a) {
  if (a.q_fmt == CSA_F32) return 0;
  int nc = attn_nchunks(a);
  if (nc <= 1 && !(attn_all_heads(a) && a.dense)) return 0;
  return (size_t)a.B * a.Q * (a.H / 16) * nc * sizeof(Partial);
}

// Dynamic LDS of a launch: the paged dense chunk's pool rows.
static size_t attn_dyn_lds(const AttnArgs& a, int cr) {
  return (a.dense && a.ent_pages.table) ? (size_t)cr * sizeof(int32_t) : 0;
}

template <int WF, int MODE>
static void launch_mfma_wl(const AttnArgs& a, int nc, int64_t nu, dim3 grid, Partial* part,
                           hipStream_t s) {
  const int cr = attn_chunk_rows(a);
  const size_t lds = attn_dyn_lds(a, cr);
  if (a.ent_fmt == CSA_BF16)
    hipLaunchKernelGGL((attn_mfma_kernel<WF, CSA_BF16, MODE>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, part);
  else if (a.ent_fmt == CSA_FP8_MX32)
    hipLaunchKernelGGL((attn_mfma_kernel<WF, CSA_FP8_MX32, MODE>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, part);
  else if (a.ent_fmt == CSA_MIX576)
    hipLaunchKernelGGL((attn_mfma_kernel<WF, CSA_MIX576, MODE>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, part);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<WF, CSA_FP4_E4M3_16, MODE>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, part);
}

template <int WF>
static void launch_mfma_w(const AttnArgs& a, int nc, int64_t nu, dim3 grid, Partial* part,
                          hipStream_t s) {
  if (attn_long_chunks(a)) launch_mfma_wl<WF, kAttnLong>(a, nc, nu, grid, part, s);
  else if (attn_whole_lists(a)) launch_mfma_wl<WF, kAttnWhole>(a, nc, nu, grid, part, s);
  else launch_mfma_wl<WF, kAttnChunks>(a, nc, nu, grid, part, s);
}

// Fewer than two work-groups per CU would leave one wave per SIMD with a
// single tile in flight: the head tiles are then split over two work-groups.
constexpr int64_t kDenseSplitBelow = 512;

template <int WF, int EF>
static void launch_all_heads_e(const AttnArgs& a, int nc, int64_t nu, Partial* part,
                               hipStream_t s) {
  const int cr0 = attn_chunk_rows(a);
  if (attn_sparse_all_heads(a)) {  // 64 heads over kSparseHsplit work-groups per item
    const int64_t items = (int64_t)nc * nu;
    if (kSparseHsplit == 1)
      hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 4, true>), dim3((unsigned)items),
                         dim3(kAttnThreads), 0, s, a, cr0, nc, nu, 1, part);
    else
      hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 4 / kSparseHsplit, true>),
                         dim3((unsigned)((items + 7) / 8 * 8 * kSparseHsplit)), dim3(kAttnThreads),
                         0, s, a, cr0, nc, nu, kSparseHsplit, part);
    return;
  }
  const int G = a.H / 16;
  const int64_t items = (int64_t)nc * nu;
  const int hsplit = (G % 2 == 0 && items < kDenseSplitBelow) ? 2 : 1;
  const int HT = G / hsplit;
  const int cr = attn_chunk_rows(a);
  const size_t lds = attn_dyn_lds(a, cr);
  const dim3 grid((unsigned)(hsplit == 1 ? items : (items + 7) / 8 * 8 * hsplit));
  switch (HT) {
    case 1: hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 1>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, hsplit, part); break;
    case 2: hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 2>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, hsplit, part); break;
    case 3: hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 3>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, hsplit, part); break;
    default: hipLaunchKernelGGL((attn_dense_all_kernel<WF, EF, 4>), grid, dim3(kAttnThreads), lds, s, a, cr, nc, nu, hsplit, part); break;
  }
}

template <int WF>
static void launch_all_heads_w(const AttnArgs& a, int nc, int64_t nu, Partial* part,
                               hipStream_t s) {
  if (a.ent_fmt == CSA_BF16) launch_all_heads_e<WF, CSA_BF16>(a, nc, nu, part, s);
  else if (a.ent_fmt == CSA_FP8_MX32) launch_all_heads_e<WF, CSA_FP8_MX32>(a, nc, nu, part, s);
  else if (a.ent_fmt == CSA_MIX576) launch_all_heads_e<WF, CSA_MIX576>(a, nc, nu, part, s);
  else launch_all_heads_e<WF, CSA_FP4_E4M3_16>(a, nc, nu, part, s);
}

static void launch_all_heads(const AttnArgs& a, int nc, int64_t nu, Partial* part, hipStream_t s) {
  if (a.win_fmt == CSA_BF16) launch_all_heads_w<CSA_BF16>(a, nc, nu, part, s);
  else if (a.win_fmt == CSA_FP8_MX32) launch_all_heads_w<CSA_FP8_MX32>(a, nc, nu, part, s);
  else launch_all_heads_w<CSA_FP4_E4M3_16>(a, nc, nu, part, s);
}

static void launch_mfma(const AttnArgs& a, int nc, int64_t nu, Partial* part, hipStream_t s) {
  // (chunk, unit) items padded to a multiple of 8, times the head groups
  const int64_t items = ((int64_t)nc * nu + 7) / 8 * 8;
  const dim3 grid((unsigned)(items * (a.H / 16)));
  if (a.win_fmt == CSA_BF16) launch_mfma_w<CSA_BF16>(a, nc, nu, grid, part, s);
  else if (a.win_fmt == CSA_FP8_MX32) launch_mfma_w<CSA_FP8_MX32>(a, nc, nu, grid, part, s);
  else launch_mfma_w<CSA_FP4_E4M3_16>(a, nc, nu, grid, part, s);
}

hipError_t launch_attention(const AttnArgs& a0, void* ws, hipStream_t s) {
  AttnArgs a = a0;
  a.win_rb = kv_row_bytes(a.win_fmt, kHeadDim);
  a.ent_rb = kv_row_bytes(a.ent_fmt, kHeadDim);
  const int64_t units = (int64_t)a.B * a.Q;
  const int nc = attn_nchunks(a);
  static_assert(kChunkHca <= kPagedIdsMax, "paged dense chunks are staged in LDS");
  if (a.q_fmt != CSA_F32 && a.dense && a.ent_pages.table && attn_chunk_rows(a) > kPagedIdsMax)
    return hipErrorInvalidConfiguration;
  // units per launch: at most 65535 (grid y of the merge) and few enough that
  // the 1-D MFMA grid stays below 2^32 work-items
  const int64_t max_items = (((int64_t)1 << 32) - 1) / ((int64_t)kAttnThreads * (a.H / 16)) - 8;
  if (a.q_fmt != CSA_F32 && nc > max_items) return hipErrorInvalidConfiguration;
  int64_t ustep = max_items / nc;
  ustep = ustep < 1 ? 1 : (ustep > 65535 ? 65535 : ustep);
  for (int64_t u0 = 0; u0 < units; u0 += ustep) {
    const unsigned nu = (unsigned)(units - u0 < ustep ? units - u0 : ustep);
    a.unit_off = u0;
    if (a.q_fmt == CSA_F32) {
      hipLaunchKernelGGL(attn_f32_kernel, dim3(a.H, nu), dim3(kAttnThreads), 0, s, a);
      continue;
    }
    const bool all_heads = attn_all_heads(a);
    if (all_heads) launch_all_heads(a, nc, nu, (Partial*)ws, s);
    else launch_mfma(a, nc, nu, (Partial*)ws, s);
    if (nc > 1 || (all_heads && a.dense))
      hipLaunchKernelGGL(attn_merge_kernel, dim3((a.H / 16) * (kHeadDim / 64), nu),
                         dim3(kAttnThreads), 0, s, a, nc,
                         (const Partial*)ws);
  }
  return hipGetLastError();
}

}  // namespace csa
