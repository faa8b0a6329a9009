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
//   * for the value product the wave writes its slice transposed into LDS
//     (rows contiguous per dim) and multiplies P (16 heads x 32 rows, bf16) by
//     it, keeping O for 16 heads x its 128 dims in 32 accumulators;
//   * each chunk leaves (m, l, O) per head; a merge kernel combines the chunks
//     in a fixed order, adds the sink, normalises and undoes the RoPE.
// Row formats are decoded exactly to bf16 on load (E4M3 x 2^e and E2M1 x E4M3
// both fit bf16's 8-bit significand).
#include "common.h"

namespace csa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kTile = 32;             // rows per tile
constexpr int kChunkCsa = 128;        // rows per work-group, top-k lists
constexpr int kChunkHca = 1024;       // rows per work-group, dense lists
constexpr int kTPitch = kTile + 8;    // LDS pitch (bf16) of the transposed slice
constexpr float kLog2e = 1.4426950408889634f;

struct RowRef {
  const uint8_t* p;  // row start, or nullptr when the row is absent
  int fmt;
};

// Resolve logical list row j of unit (b, t).
__device__ __forceinline__ RowRef resolve_row(const AttnArgs& a, int64_t unit, int64_t b, int t,
                                              int64_t j, int64_t nvis, size_t win_rb,
                                              size_t ent_rb) {
  RowRef r{nullptr, a.win_fmt};
  if (j < kWindow) {
    int64_t p = (int64_t)t - (kWindow - 1) + j;
    if (p < 0) return r;
    int64_t row;
    if (a.win_mode == CSA_WIN_RING128) {
      row = p & (kWindow - 1);
    } else {
      row = p - (int64_t)a.win_base[b];
      if (row < 0 || row >= a.win_rows) return r;
    }
    r.p = (const uint8_t*)a.win + ((size_t)b * (size_t)a.win_rows + (size_t)row) * win_rb;
    return r;
  }
  r.fmt = a.ent_fmt;
  int64_t e;
  if (a.dense) {
    e = j - kWindow;
    if (e >= nvis) return r;
  } else {
    if (j - kWindow >= a.topk) return r;
    e = a.topk_idx[unit * a.topk + (j - kWindow)];
    if (e < 0 || e >= a.Nmax) return r;
  }
  r.p = (const uint8_t*)a.entries + ((size_t)b * (size_t)a.Nmax + (size_t)e) * ent_rb;
  return r;
}

// 8 consecutive values starting at dim d0 (d0 % 8 == 0) as exact bf16.
__device__ __forceinline__ uint4 load8_bf16(const RowRef& r, int d0) {
  if (r.p == nullptr) return make_uint4(0, 0, 0, 0);
  if (r.fmt == CSA_BF16) return *(const uint4*)(r.p + 2 * d0);
  if (r.fmt == CSA_FP8_MX32) {
    uint32_t lo = *(const uint32_t*)(r.p + d0);
    uint32_t hi = *(const uint32_t*)(r.p + d0 + 4);
    float sc = exp2i((int)r.p[kHeadDim + (d0 >> 5)] - 127);
    uint4 o;
    o.x = pack_bf16x2_exact(e4m3_to_f32(lo) * sc, e4m3_to_f32(lo >> 8) * sc);
    o.y = pack_bf16x2_exact(e4m3_to_f32(lo >> 16) * sc, e4m3_to_f32(lo >> 24) * sc);
    o.z = pack_bf16x2_exact(e4m3_to_f32(hi) * sc, e4m3_to_f32(hi >> 8) * sc);
    o.w = pack_bf16x2_exact(e4m3_to_f32(hi >> 16) * sc, e4m3_to_f32(hi >> 24) * sc);
    return o;
  }
  // FP4_E4M3_16
  uint32_t c = *(const uint32_t*)(r.p + (d0 >> 1));
  float sc = e4m3_to_f32(r.p[kHeadDim / 2 + (d0 >> 4)]);
  uint4 o;
  o.x = pack_bf16x2_exact(e2m1_to_f32(c & 15u) * sc, e2m1_to_f32((c >> 4) & 15u) * sc);
  o.y = pack_bf16x2_exact(e2m1_to_f32((c >> 8) & 15u) * sc, e2m1_to_f32((c >> 12) & 15u) * sc);
  o.z = pack_bf16x2_exact(e2m1_to_f32((c >> 16) & 15u) * sc, e2m1_to_f32((c >> 20) & 15u) * sc);
  o.w = pack_bf16x2_exact(e2m1_to_f32((c >> 24) & 15u) * sc, e2m1_to_f32(c >> 28) * sc);
  return o;
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

// ------------------------------------------------------------------ MFMA kernel
__global__ void __launch_bounds__(kAttnThreads) attn_mfma_kernel(AttnArgs a, int chunk_rows,
                                                                 int nchunks, Partial* part) {
  __shared__ uint16_t Tl[4][128 * kTPitch];
  __shared__ float4 Sp[4][64][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t unit = a.unit_off + blockIdx.z;
  const int hg = blockIdx.y;
  const int chunk = blockIdx.x;
  const int64_t b = unit / a.Q;
  const int t = a.pos[unit];
  const int64_t nvis = unit_nvis(a, t);
  const int64_t list_len = kWindow + (a.dense ? nvis : (int64_t)a.topk);
  const int64_t j_begin = (int64_t)chunk * chunk_rows;
  int64_t j_end = j_begin + chunk_rows;
  if (j_end > list_len) j_end = list_len;
  const size_t win_rb = a.win_rb;
  const size_t ent_rb = a.ent_rb;
  const int rr = rope_row(a, t);
  const float zscale = a.scale * kLog2e;

  // query slice: head 16*hg + r16, dims 128*w + 32*s + 8*kq .. +8, rotated
  uint4 qa[4];
  {
    const int head = 16 * hg + r16;
    const uint16_t* qp = (const uint16_t*)a.q + (unit * a.H + head) * (int64_t)kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 128 * w + 32 * s + 8 * kq;
      uint4 raw = *(const uint4*)(qp + d0);
      if (d0 >= kHeadDim - kRopeDims) {
        float v[8];
        uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(u[j] << 16);
          v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = (d0 - (kHeadDim - kRopeDims)) / 2 + j;
          const float c = a.rope_cos[(int64_t)rr * 32 + k];
          const float sn = a.rope_sin[(int64_t)rr * 32 + k];
          const float x = v[2 * j], y = v[2 * j + 1];
          v[2 * j] = x * c - y * sn;
          v[2 * j + 1] = x * sn + y * c;
        }
        raw = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      }
      qa[s] = raw;
    }
  }

  float m_run = -INFINITY;  // running max (log2 units) for head r16
  float l_run = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint16_t* T = Tl[w];

  for (int64_t j0 = j_begin; j0 < j_end; j0 += kTile) {
    // ---- load this wave's dim slice of rows j0 + 16*rt + r16
    uint4 fr[2][4];
    uint32_t vmask = 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t j = j0 + 16 * rt + r16;
      RowRef rf{nullptr, a.win_fmt};
      if (j < j_end) rf = resolve_row(a, unit, b, t, j, nvis, win_rb, ent_rb);
      unsigned long long bal = __ballot(rf.p != nullptr);
      vmask |= (uint32_t)(bal & 0xffffull) << (16 * rt);
#pragma unroll
      for (int s = 0; s < 4; ++s) fr[rt][s] = load8_bf16(rf, 128 * w + 32 * s + 8 * kq);
    }
    __syncthreads();  // previous tile's readers of Sp / T are done

    // ---- partial logits over this wave's 128 dims
    f32x4_t sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[rt] = mfma16x16x32(as_bf16x8(fr[rt][s]), as_bf16x8(qa[s]), sacc[rt]);
    }
    Sp[w][lane][0] = make_float4(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3]);
    Sp[w][lane][1] = make_float4(sacc[1][0], sacc[1][1], sacc[1][2], sacc[1][3]);
    // ---- transposed slice for the value product: T[dim][row]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 f = fr[rt][s];
        const uint32_t u[4] = {f.x, f.y, f.z, f.w};
        const int row = 16 * rt + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * s + 8 * kq + 2 * j;
          T[d * kTPitch + row] = (uint16_t)(u[j] & 0xffffu);
          T[(d + 1) * kTPitch + row] = (uint16_t)(u[j] >> 16);
        }
      }
    __syncthreads();

    // ---- full logits: fixed-order sum of the four partials
    float z[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float4 acc = Sp[0][lane][rt];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        float4 v = Sp[ww][lane][rt];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      z[rt][0] = acc.x; z[rt][1] = acc.y; z[rt][2] = acc.z; z[rt][3] = acc.w;
    }
    // ---- online softmax for head r16 over rows 16*rt + 4*kq + r
    float tmax = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vmask >> (16 * rt + 4 * kq + r)) & 1u;
        z[rt][r] = ok ? z[rt][r] * zscale : -INFINITY;
        tmax = fmaxf(tmax, z[rt][r]);
      }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[rt][r] = (z[rt][r] == -INFINITY) ? 0.f : exp2f(z[rt][r] - m_new);
        psum += p[rt][r];
      }
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- O = alpha * O + P C over this wave's dims
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * kq + r, 64);
    const uint4 pu = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
    const bf16x8_t pa = as_bf16x8(pu);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + r16;
      const uint2 c0 = *(const uint2*)(T + d * kTPitch + 4 * kq);
      const uint2 c1 = *(const uint2*)(T + d * kTPitch + 16 + 4 * kq);
      f32x4_t acc = o[dt];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= al[r];
      o[dt] = mfma16x16x32(pa, as_bf16x8(make_uint4(c0.x, c0.y, c1.x, c1.y)), acc);
    }
  }

  // ---- chunk result
  if (nchunks > 1) {
    Partial* P = part + (unit * (a.H / 16) + hg) * (int64_t)nchunks + chunk;
    if (w == 0 && lane < 16) {
      P->m[lane] = m_run;
      P->l[lane] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        P->o[(4 * kq + r) * kHeadDim + 128 * w + 16 * dt + r16] = o[dt][r];
    return;
  }
  // single chunk: finish here
  const float sink2 = a.sink[16 * hg + r16] * kLog2e;
  const float den = (m_run == -INFINITY) ? 0.f : l_run + exp2f(sink2 - m_run);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float iv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) iv[r] = __shfl(inv, 4 * kq + r, 64);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int d = 128 * w + 16 * dt + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = o[dt][r] * iv[r];
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
__global__ void __launch_bounds__(kAttnThreads) attn_merge_kernel(AttnArgs a, int nchunks,
                                                                  const Partial* part) {
  __shared__ float sM[16], sInv[16];
  const int tid = threadIdx.x;
  const int64_t unit = a.unit_off + blockIdx.y;
  const int hg = blockIdx.x;
  const Partial* P = part + (unit * (a.H / 16) + hg) * (int64_t)nchunks;
  const int rr = rope_row(a, a.pos[unit]);
  // per head: global max, chunk-weighted sum and the sink
  if (tid < 16) {
    float M = -INFINITY;
    for (int c = 0; c < nchunks; ++c) M = fmaxf(M, P[c].m[tid]);
    float L = 0.f;
    for (int c = 0; c < nchunks; ++c) {
      const float mc = P[c].m[tid];
      L += (mc == -INFINITY) ? 0.f : P[c].l[tid] * exp2f(mc - M);
    }
    const float sink2 = a.sink[16 * hg + tid] * kLog2e;
    const float den = (M == -INFINITY) ? 0.f : L + exp2f(sink2 - M);
    sM[tid] = M;
    sInv[tid] = den > 0.f ? 1.f / den : 0.f;
  }
  __syncthreads();
  // thread -> dim pair (2*tid, 2*tid+1), all 16 heads; chunks in a fixed order
  const int d = 2 * tid;
  for (int h = 0; h < 16; ++h) {
    const float M = sM[h];
    float x = 0.f, y = 0.f;
    for (int c = 0; c < nchunks; ++c) {
      const float mc = P[c].m[h];
      if (mc == -INFINITY) continue;
      const float wgt = exp2f(mc - M);
      x += P[c].o[h * kHeadDim + d] * wgt;
      y += P[c].o[h * kHeadDim + d + 1] * wgt;
    }
    x *= sInv[h];
    y *= sInv[h];
    if (d >= kHeadDim - kRopeDims) {
      const int k = (d - (kHeadDim - kRopeDims)) >> 1;
      const float c = a.rope_cos[(int64_t)rr * 32 + k];
      const float sn = a.rope_sin[(int64_t)rr * 32 + k];
      const float nx = x * c + y * sn, ny = -x * sn + y * c;
      x = nx;
      y = ny;
    }
    store_out(a, unit, 16 * hg + h, d, x);
    store_out(a, unit, 16 * hg + h, d + 1, y);
  }
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
  for (int64_t j = 0; j < list_len; ++j) {
    RowRef rf = resolve_row(a, unit, b, t, j, nvis, win_rb, ent_rb);
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
  const float sink = a.sink[head];
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

int attn_chunk_rows(const AttnArgs& a) { return a.dense ? kChunkHca : kChunkCsa; }

int64_t attn_list_len(const AttnArgs& a) {
  return kWindow + (a.dense ? a.Nmax : (int64_t)a.topk);
}

static int attn_nchunks(const AttnArgs& a) {
  int64_t L = attn_list_len(a);
  int cr = attn_chunk_rows(a);
  return (int)((L + cr - 1) / cr);
}

size_t attn_ws_bytes(const AttnArgs& a) {
  if (a.q_fmt == CSA_F32) return 0;
  int nc = attn_nchunks(a);
  if (nc <= 1) return 0;
  return (size_t)a.B * a.Q * (a.H / 16) * nc * sizeof(Partial);
}

hipError_t launch_attention(const AttnArgs& a0, void* ws, hipStream_t s) {
  AttnArgs a = a0;
  a.win_rb = kv_row_bytes(a.win_fmt, kHeadDim);
  a.ent_rb = kv_row_bytes(a.ent_fmt, kHeadDim);
  const int64_t units = (int64_t)a.B * a.Q;
  const int nc = attn_nchunks(a);
  for (int64_t u0 = 0; u0 < units; u0 += 65535) {
    const unsigned nu = (unsigned)(units - u0 < 65535 ? units - u0 : 65535);
    a.unit_off = u0;
    if (a.q_fmt == CSA_F32) {
      hipLaunchKernelGGL(attn_f32_kernel, dim3(a.H, nu), dim3(kAttnThreads), 0, s, a);
      continue;
    }
    hipLaunchKernelGGL(attn_mfma_kernel, dim3(nc, a.H / 16, nu), dim3(kAttnThreads), 0, s, a,
                       attn_chunk_rows(a), nc, (Partial*)ws);
    if (nc > 1)
      hipLaunchKernelGGL(attn_merge_kernel, dim3(a.H / 16, nu), dim3(kAttnThreads), 0, s, a, nc,
                         (const Partial*)ws);
  }
  return hipGetLastError();
}

}  // namespace csa
