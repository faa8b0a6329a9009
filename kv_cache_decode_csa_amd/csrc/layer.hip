// The attention layer's steps on either side of the decode path, for a few
// tokens per call (decode: M = B*T <= 64 rows):
//   input  ("DeepSeek-V4 deep dive" sections 3.2, 3.3, 5.2, 3.4 notes)
//     qr  = q_norm(wq_a x)                         (held in bf16)
//     q_h = RoPE_p(wq_b qr / RMS per head)         [H][512]
//     kv  = RoPE_p(kv_norm(wkv x))  -> window ring slot p mod 128, stored
//     q_idx_h = Hadamard(RoPE_p(wq_b_idx qr))      [Hi][128]
//     w_idx   = weights_proj(x) * 128^-1/2 * Hi^-1/2
//   output (section 3.5)
//     y = wo_b [wo_a_1 o_1 ; ... ; wo_a_g o_g]     (intermediate in bf16)
// Every matrix product is a weight-streaming MFMA kernel: a wave takes 16
// weight rows over one slice of K with all of its loads in flight; slices
// write float partials that the next kernel sums in a fixed order.  The
// slicing depends on the weight shapes only, never on M, so a sequence's
// result does not depend on the batch.
#include "common.h"

namespace csa {

namespace {

// ---------------------------------------------------------------- linear
// One job: rows [0, M) of x (row stride ldx, bf16) times `groups` weight
// matrices w + g * w_gstride, each [N][K] bf16; group g reads x columns
// [g * x_gstride, + K) and writes output columns col0 + g * N + [0, N).
constexpr int kLinJobs = 4;
struct LinJob {
  const uint16_t* x;
  int64_t ldx, x_gstride;
  const uint16_t* w;
  int64_t w_gstride;
  int K, N, groups;
  int blk0;  // first work-group of this job along x
  int col0;
};
struct LinJobs {
  LinJob j[kLinJobs];
  int n;
  int ks;       // K slices (every job's K is a multiple of 32 ks)
  int M;
  int64_t ldy;  // columns of the partial-sum rows
  float* part;  // [ks][M][ldy]
};

template <int MT>
__global__ void __launch_bounds__(64) linear_kernel(LinJobs J) {
  int jb = 0;
#pragma unroll
  for (int q = 1; q < kLinJobs; ++q)
    if (q < J.n && (int)blockIdx.x >= J.j[q].blk0) jb = q;
  const LinJob& job = J.j[jb];
  const int lane = threadIdx.x;
  const int r16 = lane & 15, kq = lane >> 4;
  const int M = J.M, K = job.K, N = job.N;
  const int nblk = (N + 15) / 16;
  const int rel = (int)blockIdx.x - job.blk0;
  const int g = rel / nblk, cb = rel % nblk;
  const int n = cb * 16 + r16;
  const uint16_t* x = job.x + (int64_t)g * job.x_gstride;
  const uint16_t* wrow = job.w + (int64_t)g * job.w_gstride + (int64_t)(n < N ? n : N - 1) * K;
  constexpr int kB = MT <= 2 ? 16 : 8;
  const int L = K / J.ks;
  const int nsteps = L / 32;
  const int kb = blockIdx.y * L;
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsteps; s0 += kB) {
    u32x4_t bw[kB];
    u32x4_t ax[kB][MT];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int s = s0 + u < nsteps ? s0 + u : nsteps - 1;  // clamped repeats add zero below
      const int k = kb + 32 * s + 8 * kq;
      bw[u] = *(const u32x4_t*)(wrow + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16 < M ? 16 * mt + r16 : M - 1;
        ax[u][mt] = *(const u32x4_t*)(x + (int64_t)m * job.ldx + k);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool ok = s0 + u < nsteps;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t av = (ok && 16 * mt + r16 < M) ? ax[u][mt] : u32x4_t{0u, 0u, 0u, 0u};
        acc[mt] = mfma16x16x32(as_bf16x8(av), as_bf16x8(bw[u]), acc[mt]);
      }
    }
  }
  // D layout: lane (r16, kq) holds rows 4 kq + r of column r16
  if (n >= N) return;
  float* dst = J.part + (int64_t)blockIdx.y * M * J.ldy + job.col0 + (int64_t)g * N + n;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * kq + r;
      if (m < M) dst[(int64_t)m * J.ldy] = acc[mt][r];
    }
}

hipError_t launch_linear(const LinJobs& J, hipStream_t s) {
  int blocks = 0;
  for (int q = 0; q < J.n; ++q) blocks = J.j[q].blk0 + J.j[q].groups * ((J.j[q].N + 15) / 16);
  const dim3 grid(blocks, J.ks);
  const int mt = (J.M + 15) / 16;
  if (mt == 1) linear_kernel<1><<<grid, 64, 0, s>>>(J);
  else if (mt == 2) linear_kernel<2><<<grid, 64, 0, s>>>(J);
  else if (mt == 3) linear_kernel<3><<<grid, 64, 0, s>>>(J);
  else linear_kernel<4><<<grid, 64, 0, s>>>(J);
  return hipGetLastError();
}

// Slices of K: enough work-groups to cover the chip (about 2,048 waves), at
// most max_ks, each slice a multiple of 32 wide.  Depends on the weight
// shapes only.
int pick_slices(int blocks, int K, int max_ks = 16) {
  int ks = 1;
  while (ks < max_ks && blocks * ks < 2048 && K % (64 * ks) == 0) ks *= 2;
  return ks;
}

void add_job(LinJobs& J, const void* x, int64_t ldx, int64_t x_gstride, const void* w,
             int64_t w_gstride, int K, int N, int groups, int col0) {
  LinJob& j = J.j[J.n];
  j.x = (const uint16_t*)x;
  j.ldx = ldx;
  j.x_gstride = x_gstride;
  j.w = (const uint16_t*)w;
  j.w_gstride = w_gstride;
  j.K = K;
  j.N = N;
  j.groups = groups;
  j.col0 = col0;
  j.blk0 = J.n == 0 ? 0 : J.j[J.n - 1].blk0 + J.j[J.n - 1].groups * ((J.j[J.n - 1].N + 15) / 16);
  ++J.n;
}

int job_blocks(const LinJobs& J) {
  const LinJob& l = J.j[J.n - 1];
  return l.blk0 + l.groups * ((l.N + 15) / 16);
}

// ---------------------------------------------------------------- epilogues
constexpr int kThreads = 256;

// Sum of the ks (<= kMaxSlices) partials of element i, added in slice order;
// the loads are independent, so they are in flight together.
constexpr int kMaxSlices = 16;
__device__ __forceinline__ float slice_sum(const float* part, int ks, int64_t stride, int64_t i) {
  float v[kMaxSlices];
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s) v[s] = s < ks ? part[s * stride + i] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int s = 1; s < kMaxSlices; ++s)
    if (s < ks) acc += v[s];
  return acc;
}

constexpr int kMaxRank = 2048;  // largest q_rank

struct InArgs {
  const float* part;  // [ks][M][ldy]: latent | window entry | head weights
  int ks, M, T;
  int64_t ldy;
  int QR, Hi;
  const float* q_norm;
  const float* kv_norm;
  float eps, w_scale;
  const int32_t* pos;  // [M]
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_rows;
  uint16_t* qr;        // [M][QR] bf16
  float* w_idx;        // [M][Hi]
  uint8_t* win;        // [B][128][win_rb]
  int win_fmt;
  size_t win_rb;
};

__device__ __forceinline__ int64_t rope_row(int64_t p, int64_t rows) {
  return p < 0 ? 0 : (p >= rows ? rows - 1 : p);
}

// One work-group per row m: latent RMSNorm -> bf16; window entry RMSNorm ->
// RoPE -> stored into ring slot pos mod 128; head weights scaled.  Every load
// that does not depend on another is issued first, so the kernel waits for
// memory about twice (the loads, then the rotation factors at the position).
template <int TT>
__global__ void __launch_bounds__(TT) layer_in_kernel(InArgs a) {
  static_assert(TT == 256 || TT == 512, "4 or 8 waves");
  constexpr int kL = kMaxRank / TT;
  constexpr int kW = kHeadDim / TT;  // window dims per thread
  __shared__ float red[2][TT / 64];
  __shared__ float z[kHeadDim];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int64_t stride = (int64_t)a.M * a.ldy;
  const float* row = a.part + (int64_t)m * a.ldy;
  const int64_t p = a.pos[m];
  float lv[kL], gq[kL];
#pragma unroll
  for (int u = 0; u < kL; ++u) {
    const int c = tid + u * TT;
    lv[u] = c < a.QR ? slice_sum(row, a.ks, stride, c) : 0.f;
    gq[u] = c < a.QR ? a.q_norm[c] : 0.f;
  }
  float v[kW], gk[kW];
#pragma unroll
  for (int u = 0; u < kW; ++u) {
    v[u] = slice_sum(row, a.ks, stride, a.QR + tid + u * TT);
    gk[u] = a.kv_norm[tid + u * TT];
  }
  const float wv = tid < a.Hi ? slice_sum(row, a.ks, stride, a.QR + kHeadDim + tid) : 0.f;
  // rotation factors of this thread's last window dim (the rotated dims
  // 448..511 are all last dims: tid + (kW - 1) TT >= 448)
  const int64_t rr = rope_row(p, a.rope_rows);
  const int c1 = tid + (kW - 1) * TT;
  float cs = 1.f, sn = 0.f;
  if (c1 >= kHeadDim - kRopeDims) {
    const int k = (c1 - (kHeadDim - kRopeDims)) >> 1;
    cs = a.rope_cos[rr * 32 + k];
    sn = a.rope_sin[rr * 32 + k];
  }
  // both sums of squares in one pass
  float sq = 0.f;
#pragma unroll
  for (int u = 0; u < kL; ++u) sq += lv[u] * lv[u];
  float sk = 0.f;
#pragma unroll
  for (int u = 0; u < kW; ++u) sk += v[u] * v[u];
  sq = wave_sum(sq);
  sk = wave_sum(sk);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sq;
    red[1][tid >> 6] = sk;
  }
  __syncthreads();
  // wave sums, pairwise in a fixed order
  float tq = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  float tk = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  if (TT == 512) {
    tq = tq + ((red[0][4] + red[0][5]) + (red[0][6] + red[0][7]));
    tk = tk + ((red[1][4] + red[1][5]) + (red[1][6] + red[1][7]));
  }
  const float inv_q = 1.0f / sqrtf(tq / (float)a.QR + a.eps);
  const float inv_k = 1.0f / sqrtf(tk / (float)kHeadDim + a.eps);
#pragma unroll
  for (int u = 0; u < kL; ++u) {
    const int c = tid + u * TT;
    if (c < a.QR) a.qr[(int64_t)m * a.QR + c] = f32_to_bf16(lv[u] * inv_q * gq[u]);
  }
  if (tid < a.Hi) a.w_idx[(int64_t)m * a.Hi + tid] = wv * a.w_scale;
#pragma unroll
  for (int u = 0; u < kW; ++u) z[tid + u * TT] = v[u] * inv_k * gk[u];
  __syncthreads();
  if (p < 0) return;
  const int b = m / a.T;
  uint8_t* dst = a.win + ((int64_t)b * kWindow + p % kWindow) * a.win_rb;
#pragma unroll
  for (int u = 0; u < kW; ++u) {
    const int c = tid + u * TT;
    float out = z[c];
    if (c >= kHeadDim - kRopeDims) {
      const float pv = z[c ^ 1];
      out = (c & 1) ? (pv * sn + out * cs) : (out * cs - pv * sn);
    }
    if (a.win_fmt == CSA_F32) ((float*)dst)[c] = out;
    else if (a.win_fmt == CSA_BF16) ((uint16_t*)dst)[c] = f32_to_bf16(out);
    else store_elem(a.win_fmt, out, c, kHeadDim, true, dst);
  }
}

struct QArgs {
  const float* part;  // [ks][M][ldy]: H heads of 512 | Hi heads of 128
  int ks, M, H, Hi;
  int64_t ldy;
  float eps;
  const int32_t* pos;
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_rows;
  uint16_t* q;      // [M][H][512] bf16
  uint16_t* q_idx;  // [M][Hi][128] bf16
};

// One wave per (row, head).  Query heads: lane l holds dims 8l .. 8l+7, RMS
// over the head; they are written un-rotated, since the attention calls rotate
// q at the query's position themselves.  Index heads: lane l holds dims l and
// l + 64; RoPE pairs across lanes l, l^1 of the upper half; Sylvester Hadamard
// butterflies (stride 64 in-lane, then strides 32..1 across lanes) scaled by
// 128^-1/2.
__global__ void __launch_bounds__(kThreads) layer_q_kernel(QArgs a) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (head >= a.H + a.Hi) return;
  const int64_t stride = (int64_t)a.M * a.ldy;
  const float* row = a.part + (int64_t)m * a.ldy;
  if (head < a.H) {
    float v[8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = slice_sum(row, a.ks, stride, (int64_t)head * kHeadDim + 8 * lane + j);
      ss += v[j] * v[j];
    }
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)kHeadDim + a.eps);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(v[2 * j] * inv, v[2 * j + 1] * inv);
    *(u32x4_t*)(a.q + ((int64_t)m * a.H + head) * kHeadDim + 8 * lane) = o;
    return;
  }
  const int64_t rr = rope_row(a.pos[m], a.rope_rows);
  const int h = head - a.H;
  const int64_t base = (int64_t)a.H * kHeadDim + (int64_t)h * kIndexDim;
  const float cs = a.rope_cos[rr * 32 + (lane >> 1)], sn = a.rope_sin[rr * 32 + (lane >> 1)];
  float lo = slice_sum(row, a.ks, stride, base + lane);
  float hi = slice_sum(row, a.ks, stride, base + lane + 64);
  {  // RoPE on dims 64..127: dim 64 + lane pairs with 64 + (lane ^ 1), pair lane / 2
    const float pv = shfl_xor_f(hi, 1);
    hi = (lane & 1) ? (pv * sn + hi * cs) : (hi * cs - pv * sn);
  }
  {
    const float s = lo + hi, d = lo - hi;
    lo = s;
    hi = d;
  }
#pragma unroll
  for (int st = 32; st >= 1; st >>= 1) {
    const float plo = shfl_xor_f(lo, st), phi = shfl_xor_f(hi, st);
    const bool up = lane & st;
    lo = up ? plo - lo : lo + plo;
    hi = up ? phi - hi : hi + phi;
  }
  const float sc = 1.0f / sqrtf((float)kIndexDim);
  uint16_t* dst = a.q_idx + ((int64_t)m * a.Hi + h) * kIndexDim;
  dst[lane] = f32_to_bf16(lo * sc);
  dst[lane + 64] = f32_to_bf16(hi * sc);
}

// Sum of ks slices -> out (float32 or bf16), one element per thread.
__global__ void __launch_bounds__(kThreads) slice_sum_kernel(const float* __restrict__ part, int ks,
                                                             int64_t n, void* out, int out_fmt) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float v = slice_sum(part, ks, n, i);
  if (out_fmt == CSA_F32) ((float*)out)[i] = v;
  else ((uint16_t*)out)[i] = f32_to_bf16(v);
}

// ---------------------------------------------------------------- workspace
struct InPlan {
  LinJobs a, b;
  size_t off_part_a, off_qr, off_part_b, total;
};

InPlan plan_input(const csa_layer_weights* w, int M) {
  InPlan p{};
  const int64_t lda = (int64_t)w->q_rank + kHeadDim + w->Hi;
  p.a.M = M;
  p.a.ldy = lda;
  add_job(p.a, nullptr, w->dim, 0, w->wq_a, 0, w->dim, w->q_rank, 1, 0);
  add_job(p.a, nullptr, w->dim, 0, w->wkv, 0, w->dim, kHeadDim, 1, w->q_rank);
  if (w->Hi > 0) add_job(p.a, nullptr, w->dim, 0, w->w_proj, 0, w->dim, w->Hi, 1, w->q_rank + kHeadDim);
  // few slices: one work-group per row sums them in the epilogue
  p.a.ks = pick_slices(job_blocks(p.a), w->dim, 4);
  const int64_t ldb = (int64_t)w->H * kHeadDim + (int64_t)w->Hi * kIndexDim;
  p.b.M = M;
  p.b.ldy = ldb;
  add_job(p.b, nullptr, w->q_rank, 0, w->wq_b, 0, w->q_rank, w->H * kHeadDim, 1, 0);
  if (w->Hi > 0)
    add_job(p.b, nullptr, w->q_rank, 0, w->wq_b_idx, 0, w->q_rank, w->Hi * kIndexDim, 1,
            w->H * kHeadDim);
  p.b.ks = pick_slices(job_blocks(p.b), w->q_rank);
  size_t off = 0;
  p.off_part_a = off;
  off = align_up(off + (size_t)p.a.ks * M * lda * 4, 256);
  p.off_qr = off;
  off = align_up(off + (size_t)M * w->q_rank * 2, 256);
  p.off_part_b = off;
  off = align_up(off + (size_t)p.b.ks * M * ldb * 4, 256);
  p.total = off;
  return p;
}

struct OutPlan {
  LinJobs a, b;
  size_t off_part_a, off_mid, off_part_b, total;
};

OutPlan plan_output(const csa_layer_weights* w, int M) {
  OutPlan p{};
  const int gw = w->H / w->groups * kHeadDim;  // x columns per group
  const int mid = w->groups * w->o_rank;
  p.a.M = M;
  p.a.ldy = mid;
  add_job(p.a, nullptr, (int64_t)w->H * kHeadDim, gw, w->wo_a, (int64_t)w->o_rank * gw, gw,
          w->o_rank, w->groups, 0);
  p.a.ks = pick_slices(job_blocks(p.a), gw);
  p.b.M = M;
  p.b.ldy = w->dim;
  add_job(p.b, nullptr, mid, 0, w->wo_b, 0, mid, w->dim, 1, 0);
  p.b.ks = pick_slices(job_blocks(p.b), mid);
  size_t off = 0;
  p.off_part_a = off;
  off = align_up(off + (size_t)p.a.ks * M * mid * 4, 256);
  p.off_mid = off;
  off = align_up(off + (size_t)M * mid * 2, 256);
  p.off_part_b = off;
  off = align_up(off + (size_t)p.b.ks * M * w->dim * 4, 256);
  p.total = off;
  return p;
}

}  // namespace

size_t layer_input_ws_bytes(const csa_layer_weights* w, int M) { return plan_input(w, M).total; }
size_t layer_output_ws_bytes(const csa_layer_weights* w, int M) { return plan_output(w, M).total; }

hipError_t launch_layer_input(const csa_layer_weights* w, const void* x, const int32_t* pos, int B,
                              int T, const float* rope_cos, const float* rope_sin,
                              int64_t rope_rows, void* q, void* q_idx, float* w_idx, void* win,
                              int win_fmt, size_t win_rb, void* ws, hipStream_t s) {
  const int M = B * T;
  InPlan p = plan_input(w, M);
  uint8_t* base = (uint8_t*)ws;
  for (int i = 0; i < p.a.n; ++i) p.a.j[i].x = (const uint16_t*)x;
  p.a.part = (float*)(base + p.off_part_a);
  uint16_t* qr = (uint16_t*)(base + p.off_qr);
  for (int i = 0; i < p.b.n; ++i) p.b.j[i].x = qr;
  p.b.part = (float*)(base + p.off_part_b);
  hipError_t e = launch_linear(p.a, s);
  if (e != hipSuccess) return e;
  InArgs ia{};
  ia.part = p.a.part;
  ia.ks = p.a.ks;
  ia.M = M;
  ia.T = T;
  ia.ldy = p.a.ldy;
  ia.QR = w->q_rank;
  ia.Hi = w->Hi;
  ia.q_norm = w->q_norm;
  ia.kv_norm = w->kv_norm;
  ia.eps = w->eps;
  ia.w_scale = w->Hi > 0 ? (float)(1.0 / sqrt((double)kIndexDim * (double)w->Hi)) : 0.f;
  ia.pos = pos;
  ia.rope_cos = rope_cos;
  ia.rope_sin = rope_sin;
  ia.rope_rows = rope_rows;
  ia.qr = qr;
  ia.w_idx = w_idx;
  ia.win = (uint8_t*)win;
  ia.win_fmt = win_fmt;
  ia.win_rb = win_rb;
  layer_in_kernel<512><<<M, 512, 0, s>>>(ia);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_linear(p.b, s);
  if (e != hipSuccess) return e;
  QArgs qa{};
  qa.part = p.b.part;
  qa.ks = p.b.ks;
  qa.M = M;
  qa.H = w->H;
  qa.Hi = w->Hi;
  qa.ldy = p.b.ldy;
  qa.eps = w->eps;
  qa.pos = pos;
  qa.rope_cos = rope_cos;
  qa.rope_sin = rope_sin;
  qa.rope_rows = rope_rows;
  qa.q = (uint16_t*)q;
  qa.q_idx = (uint16_t*)q_idx;
  layer_q_kernel<<<dim3(M, (w->H + w->Hi + 3) / 4), kThreads, 0, s>>>(qa);
  return hipGetLastError();
}

hipError_t launch_layer_output(const csa_layer_weights* w, const void* o, int M, void* y,
                               int y_fmt, void* ws, hipStream_t s) {
  OutPlan p = plan_output(w, M);
  uint8_t* base = (uint8_t*)ws;
  p.a.j[0].x = (const uint16_t*)o;
  p.a.part = (float*)(base + p.off_part_a);
  uint16_t* mid = (uint16_t*)(base + p.off_mid);
  p.b.j[0].x = mid;
  p.b.part = (float*)(base + p.off_part_b);
  hipError_t e = launch_linear(p.a, s);
  if (e != hipSuccess) return e;
  const int64_t nm = (int64_t)M * p.a.ldy;
  slice_sum_kernel<<<(nm + kThreads - 1) / kThreads, kThreads, 0, s>>>(p.a.part, p.a.ks, nm, mid,
                                                                       CSA_BF16);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_linear(p.b, s);
  if (e != hipSuccess) return e;
  const int64_t ny = (int64_t)M * w->dim;
  slice_sum_kernel<<<(ny + kThreads - 1) / kThreads, kThreads, 0, s>>>(p.b.part, p.b.ks, ny, y,
                                                                       y_fmt);
  return hipGetLastError();
}

}  // namespace csa
