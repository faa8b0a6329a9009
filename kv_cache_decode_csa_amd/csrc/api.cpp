// C entry points of libcsa: host-side validation, workspace sizing and
// dispatch to the kernel launchers.  Nothing here touches device memory until
// every argument has been checked.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "csa_internal.h"

using namespace csa;

namespace {

thread_local char g_detail[512] = "";

csa_status fail(csa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return code;
}

csa_status ok() {
  g_detail[0] = 0;
  return CSA_OK;
}

csa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSA_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...)                   \
  do {                                             \
    if (!(cond)) return fail(code, __VA_ARGS__);   \
  } while (0)

#define REQUIRE_PTR(p) \
  REQUIRE((p) != nullptr && aligned16(p), CSA_EINVAL, "%s must be a non-null 16-byte aligned pointer", #p)

bool valid_fmt(int f) { return f >= CSA_F32 && f <= CSA_MIX576; }
// cache rows that attention and the compressor read or write (MXFP4-MX32 is
// an index-key format)
bool row_fmt(int f) { return f >= CSA_F32 && f <= CSA_FP4_E4M3_16; }

}  // namespace

namespace csa {
csa_status set_error(csa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace csa

extern "C" {

const char* csa_strerror(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_EINVAL: return "invalid argument";
    case CSA_EUNSUPPORTED: return "unsupported format or shape";
    case CSA_EWORKSPACE: return "workspace too small";
    case CSA_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* csa_last_error_detail(void) { return g_detail; }

size_t kv_row_bytes(int fmt, int dim) {
  if (dim <= 0) return 0;
  switch (fmt) {
    case CSA_F32: return (size_t)dim * 4;
    case CSA_BF16: return (size_t)dim * 2;
    case CSA_FP8_MX32: return dim % 32 ? 0 : (size_t)dim + dim / 32;
    case CSA_FP4_E4M3_16: return dim % 32 ? 0 : (size_t)dim / 2 + dim / 16;
    case CSA_FP4_MX32: return dim % 32 ? 0 : (size_t)dim / 2 + dim / 32;
    case CSA_MIX576: return dim == 512 ? 592 : 0;
    default: return 0;
  }
}

// ---------------------------------------------------------------- RoPE table
csa_status csa_rope_table(double theta, double yarn_factor, int64_t yarn_orig_len,
                          double beta_fast, double beta_slow, int64_t rows, float* cos_out,
                          float* sin_out, csa_stream_t stream) {
  REQUIRE_PTR(cos_out);
  REQUIRE_PTR(sin_out);
  REQUIRE(rows >= 1, CSA_EINVAL, "rows must be >= 1 (got %lld)", (long long)rows);
  REQUIRE(theta > 1.0 && isfinite(theta), CSA_EINVAL, "theta must be finite and > 1");
  REQUIRE(!(yarn_factor > 0) || (yarn_orig_len > 0 && beta_fast > 0 && beta_slow > 0),
          CSA_EINVAL, "YaRN needs yarn_orig_len > 0 and positive betas");
  const int npairs = kRopeDims / 2;
  double omega[kRopeDims / 2];
  for (int k = 0; k < npairs; ++k) omega[k] = pow(theta, -2.0 * k / kRopeDims);
  if (yarn_factor > 0) {
    // correction range of section 9.1: dims * ln(L0 / (2 pi beta)) / (2 ln theta)
    auto corr = [&](double beta) {
      return kRopeDims * log((double)yarn_orig_len / (2.0 * M_PI * beta)) / (2.0 * log(theta));
    };
    double lo = floor(corr(beta_fast)), hi = ceil(corr(beta_slow));
    if (lo < 0) lo = 0;
    if (hi > npairs - 1) hi = npairs - 1;
    if (hi == lo) hi += 0.001;
    for (int k = 0; k < npairs; ++k) {
      double ramp = (k - lo) / (hi - lo);
      ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
      double smooth = 1.0 - ramp;
      omega[k] = omega[k] / yarn_factor * (1.0 - smooth) + omega[k] * smooth;
    }
  }
  return launched(launch_rope_table(omega, rows, cos_out, sin_out, (hipStream_t)stream),
                  "rope_table");
}

// ---------------------------------------------------------------- codec
csa_status kv_quantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                       int dim, csa_stream_t stream) {
  REQUIRE(rows >= 0, CSA_EINVAL, "rows must be >= 0");
  REQUIRE(dim > 0 && dim % 32 == 0, CSA_EINVAL, "dim must be a positive multiple of 32 (got %d)", dim);
  REQUIRE(src_fmt == CSA_F32 || src_fmt == CSA_BF16, CSA_EUNSUPPORTED, "src_fmt must be F32 or BF16");
  REQUIRE(valid_fmt(dst_fmt), CSA_EUNSUPPORTED, "unknown dst_fmt %d", dst_fmt);
  REQUIRE(dst_fmt != CSA_FP8_MX32 || dim % 128 == 0, CSA_EUNSUPPORTED,
          "FP8_MX32 rows need dim % 128 == 0 (4-byte aligned rows)");
  REQUIRE(dst_fmt != CSA_FP4_MX32 || dim % 128 == 0, CSA_EUNSUPPORTED,
          "FP4_MX32 rows need dim % 128 == 0 (4-byte aligned rows)");
  REQUIRE(dst_fmt != CSA_MIX576 || dim == 512, CSA_EUNSUPPORTED, "MIX576 rows need dim == 512");
  if (rows == 0) return ok();
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  return launched(launch_quantize(src, src_fmt, dst, dst_fmt, rows, dim, (hipStream_t)stream),
                  "kv_quantize");
}

csa_status kv_dequantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                         int dim, csa_stream_t stream) {
  REQUIRE(rows >= 0, CSA_EINVAL, "rows must be >= 0");
  REQUIRE(dim > 0 && dim % 32 == 0, CSA_EINVAL, "dim must be a positive multiple of 32 (got %d)", dim);
  REQUIRE(valid_fmt(src_fmt), CSA_EUNSUPPORTED, "unknown src_fmt %d", src_fmt);
  REQUIRE(dst_fmt == CSA_F32 || dst_fmt == CSA_BF16, CSA_EUNSUPPORTED, "dst_fmt must be F32 or BF16");
  REQUIRE(src_fmt != CSA_FP8_MX32 || dim % 128 == 0, CSA_EUNSUPPORTED,
          "FP8_MX32 rows need dim % 128 == 0 (4-byte aligned rows)");
  REQUIRE(src_fmt != CSA_FP4_MX32 || dim % 128 == 0, CSA_EUNSUPPORTED,
          "FP4_MX32 rows need dim % 128 == 0 (4-byte aligned rows)");
  REQUIRE(src_fmt != CSA_MIX576 || dim == 512, CSA_EUNSUPPORTED, "MIX576 rows need dim == 512");
  if (rows == 0) return ok();
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  return launched(launch_dequantize(src, src_fmt, dst, dst_fmt, rows, dim, (hipStream_t)stream),
                  "kv_dequantize");
}

// ---------------------------------------------------------------- block cache
// Validates a block-table descriptor (entries per block a power of two in
// [min_entries, 1024]) and turns it into the kernels' PageMap.
static csa_status page_map(const int32_t* table, int64_t max_blocks, int block_entries,
                           int64_t pool_blocks, int min_entries, PageMap* out) {
  REQUIRE_PTR(table);
  REQUIRE(max_blocks >= 1, CSA_EINVAL, "max_blocks must be >= 1");
  REQUIRE(pool_blocks >= 1 && pool_blocks <= INT32_MAX, CSA_EINVAL,
          "pool_blocks must be in [1, 2^31 - 1]");
  REQUIRE(block_entries >= min_entries && block_entries <= 1024 &&
              (block_entries & (block_entries - 1)) == 0,
          CSA_EINVAL, "block_entries must be a power of two in [%d, 1024] (got %d)", min_entries,
          block_entries);
  REQUIRE(max_blocks <= ((int64_t)1 << 30) / block_entries, CSA_EINVAL,
          "max_blocks * block_entries must be <= 2^30");
  int shift = 0;
  while ((1 << shift) < block_entries) ++shift;
  *out = PageMap{table, max_blocks, pool_blocks, shift};
  return CSA_OK;
}

static csa_status page_map(const csa_block_table* t, int min_entries, PageMap* out) {
  REQUIRE(t != nullptr, CSA_EINVAL, "block table descriptor must not be null");
  return page_map(t->table, t->max_blocks, t->block_entries, t->pool_blocks, min_entries, out);
}

// ---------------------------------------------------------------- compressor
static csa_status check_compress(const csa_compress_args* a) {
  REQUIRE(a != nullptr, CSA_EINVAL, "args must not be null");
  REQUIRE(a->B >= 1 && a->T >= 1, CSA_EINVAL, "B and T must be >= 1");
  REQUIRE(a->dim >= 32 && a->dim % 32 == 0, CSA_EINVAL, "dim must be a positive multiple of 32");
  REQUIRE(a->ratio == 1 || a->ratio == 2 || a->ratio == 4 || a->ratio == 128, CSA_EUNSUPPORTED,
          "ratio must be 1, 2, 4 or 128 (got %d)", a->ratio);
  REQUIRE(a->head_dim == 128 || a->head_dim == 512, CSA_EUNSUPPORTED, "head_dim must be 128 or 512");
  REQUIRE(!a->rotate || a->head_dim == 128, CSA_EUNSUPPORTED, "rotate needs head_dim 128");
  REQUIRE(a->x_fmt == CSA_F32 || a->x_fmt == CSA_BF16, CSA_EUNSUPPORTED, "x_fmt must be F32 or BF16");
  REQUIRE(a->w_fmt == CSA_F32 || a->w_fmt == CSA_BF16, CSA_EUNSUPPORTED, "w_fmt must be F32 or BF16");
  REQUIRE(row_fmt(a->entry_fmt) || (a->entry_fmt == CSA_FP4_MX32 && a->head_dim == 128) ||
              (a->entry_fmt == CSA_MIX576 && a->head_dim == 512),
          CSA_EUNSUPPORTED, "entry_fmt must be F32, BF16, FP8_MX32, FP4_E4M3_16, FP4_MX32 "
          "for 128-d index keys, or MIX576 for 512-d entries");
  REQUIRE(a->rope_rows >= 1, CSA_EINVAL, "rope_rows must be >= 1");
  REQUIRE(a->entries_cap >= 0, CSA_EINVAL, "entries_cap must be >= 0");
  REQUIRE(a->eps >= 0 && isfinite(a->eps), CSA_EINVAL, "eps must be finite and >= 0");
  REQUIRE_PTR(a->x);
  REQUIRE_PTR(a->w_kv);
  REQUIRE_PTR(a->w_gate);
  REQUIRE_PTR(a->ape);
  REQUIRE_PTR(a->norm_w);
  REQUIRE_PTR(a->rope_cos);
  REQUIRE_PTR(a->rope_sin);
  REQUIRE_PTR(a->start_pos);
  REQUIRE_PTR(a->kv_state);
  REQUIRE_PTR(a->score_state);
  if (a->block_table) {
    PageMap pm;
    csa_status st = page_map(a->block_table, a->max_blocks, a->block_entries, a->pool_blocks, 1,
                             &pm);
    if (st != CSA_OK) return st;
    REQUIRE_PTR(a->entries);
  } else if (a->entries_cap > 0) {
    REQUIRE_PTR(a->entries);
  }
  if (a->state_slot) {
    REQUIRE_PTR(a->state_slot);
    REQUIRE(a->state_slots >= 1 && a->state_slots <= INT32_MAX, CSA_EINVAL,
            "state_slots must be in [1, 2^31 - 1]");
  }
  return CSA_OK;
}

size_t csa_compress_workspace_size(const csa_compress_args* a) {
  if (check_compress(a) != CSA_OK) return 0;
  return compress_ws_bytes(a);
}

csa_status csa_compress(const csa_compress_args* a, void* ws, size_t ws_bytes,
                        csa_stream_t stream) {
  csa_status st = check_compress(a);
  if (st != CSA_OK) return st;
  size_t need = compress_ws_bytes(a);
  REQUIRE(need == 0 || (ws != nullptr && aligned16(ws) && ws_bytes >= need), CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  return launched(launch_compress(a, ws, (hipStream_t)stream), "csa_compress");
}

size_t csa_compress_many_workspace_size(const csa_compress_args* a, int n) {
  if (a == nullptr || n < 1 || n > 4) return 0;
  for (int i = 0; i < n; ++i)
    if (check_compress(&a[i]) != CSA_OK) return 0;
  return compress_many_ws_bytes(a, n);
}

csa_status csa_compress_many(const csa_compress_args* a, int n, void* ws, size_t ws_bytes,
                             csa_stream_t stream) {
  REQUIRE(a != nullptr, CSA_EINVAL, "args must not be null");
  REQUIRE(n >= 1 && n <= 4, CSA_EUNSUPPORTED, "n must be in [1, 4]");
  for (int i = 0; i < n; ++i) {
    csa_status st = check_compress(&a[i]);
    if (st != CSA_OK) return st;
  }
  size_t need = compress_many_ws_bytes(a, n);
  REQUIRE(need == 0 || (ws != nullptr && aligned16(ws) && ws_bytes >= need), CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  return launched(launch_compress_many(a, n, ws, (hipStream_t)stream), "csa_compress_many");
}

// ---------------------------------------------------------------- top-k
size_t csa_topk_workspace_size(int64_t R, int64_t ld, int topk) {
  (void)ld;
  (void)topk;
  if (R < 1) return 0;
  return topk_ws_bytes(R);
}

csa_status csa_topk(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld, int topk,
                    int32_t* out_idx, void* ws, size_t ws_bytes, csa_stream_t stream) {
  REQUIRE(R >= 0, CSA_EINVAL, "R must be >= 0");
  REQUIRE(ld >= 1, CSA_EINVAL, "ld must be >= 1");
  REQUIRE(topk >= 1 && topk <= kTopkMax, CSA_EUNSUPPORTED, "topk must be in [1, %d] (got %d)",
          kTopkMax, topk);
  if (R == 0) return ok();
  REQUIRE_PTR(scores);
  REQUIRE_PTR(n_valid);
  REQUIRE_PTR(out_idx);
  size_t need = topk_ws_bytes(R);
  REQUIRE(ws != nullptr && aligned16(ws) && ws_bytes >= need, CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  TopkWs w = topk_ws_carve(ws, R);
  hipError_t e = launch_topk_clear(w, R, s);
  if (e == hipSuccess) e = launch_topk_hist(scores, n_valid, R, ld, w, s);
  if (e == hipSuccess) e = launch_topk_select(scores, n_valid, R, ld, topk, out_idx, w, s);
  return launched(e, "csa_topk");
}

size_t csa_index_topk_workspace_size(int B, int Q, int64_t Nmax, int topk) {
  (void)topk;
  if (B < 1 || Q < 1 || Nmax < 1) return 0;
  int64_t R = (int64_t)B * Q;
  return align_up(topk_ws_bytes(R), 256) + align_up((size_t)R * 4, 256) +
         align_up((size_t)R * (size_t)Nmax * 4, 256);
}

static csa_status index_topk(const void* q_idx, int q_fmt, const float* w_idx, const void* k_idx,
                          int k_fmt, const int32_t* pos, int ratio, int B, int Q, int Hi,
                          int64_t Nmax, int topk, int32_t* out_idx, float* out_scores, void* ws,
                          size_t ws_bytes, csa_stream_t stream, int bf16_scores,
                          PageMap pm = PageMap{nullptr, 0, 0, 0}) {
  REQUIRE(B >= 1 && Q >= 1, CSA_EINVAL, "B and Q must be >= 1");
  REQUIRE(Nmax >= 1 && Nmax <= (int64_t)1 << 30, CSA_EINVAL, "Nmax must be in [1, 2^30]");
  REQUIRE(ratio >= 1, CSA_EINVAL, "ratio must be >= 1");
  REQUIRE(topk >= 1 && topk <= kTopkMax, CSA_EUNSUPPORTED, "topk must be in [1, %d]", kTopkMax);
  REQUIRE(Hi >= 1, CSA_EINVAL, "Hi must be >= 1");
  if (k_fmt == CSA_F32) {
    REQUIRE(q_fmt == CSA_F32, CSA_EUNSUPPORTED, "F32 keys need F32 queries");
    REQUIRE(Hi <= 128, CSA_EUNSUPPORTED, "Hi must be <= 128");
  } else {
    REQUIRE(k_fmt == CSA_BF16 || k_fmt == CSA_FP8_MX32 || k_fmt == CSA_FP4_MX32,
            CSA_EUNSUPPORTED, "k_fmt must be F32, BF16, FP8_MX32 or FP4_MX32");
    REQUIRE(q_fmt == CSA_BF16 || (q_fmt == CSA_FP4_MX32 && k_fmt == CSA_FP4_MX32),
            CSA_EUNSUPPORTED,
            "BF16/FP8 keys need BF16 queries; FP4_MX32 keys take BF16 or FP4_MX32 queries");
    REQUIRE(Hi % 16 == 0 && Hi <= 128, CSA_EUNSUPPORTED, "Hi must be a multiple of 16, <= 128");
  }
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(w_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(out_idx);
  if (out_scores) REQUIRE_PTR(out_scores);
  size_t need = csa_index_topk_workspace_size(B, Q, Nmax, topk);
  REQUIRE(ws != nullptr && aligned16(ws) && ws_bytes >= need, CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  int64_t R = (int64_t)B * Q;
  char* p = (char*)ws;
  TopkWs w = topk_ws_carve(p, R);
  p += align_up(topk_ws_bytes(R), 256);
  int32_t* nvis = (int32_t*)p;
  p += align_up((size_t)R * 4, 256);
  float* scores = out_scores ? out_scores : (float*)p;
  hipError_t e = launch_topk_clear(w, R, s);
  if (e == hipSuccess)
    e = launch_index_scores(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax,
                            scores, nvis, w, bf16_scores, s, pm);
  if (e == hipSuccess) e = launch_topk_select(scores, nvis, R, Nmax, topk, out_idx, w, s);
  return launched(e, "csa_index_topk");
}

csa_status csa_index_topk(const void* q_idx, int q_fmt, const float* w_idx, const void* k_idx,
                          int k_fmt, const int32_t* pos, int ratio, int B, int Q, int Hi,
                          int64_t Nmax, int topk, int32_t* out_idx, float* out_scores, void* ws,
                          size_t ws_bytes, csa_stream_t stream) {
  return index_topk(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk, out_idx,
                    out_scores, ws, ws_bytes, stream, 0);
}

csa_status csa_index_topk_bf16(const void* q_idx, int q_fmt, const float* w_idx,
                               const void* k_idx, int k_fmt, const int32_t* pos, int ratio,
                               int B, int Q, int Hi, int64_t Nmax, int topk, int32_t* out_idx,
                               float* out_scores, void* ws, size_t ws_bytes,
                               csa_stream_t stream) {
  return index_topk(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk, out_idx,
                    out_scores, ws, ws_bytes, stream, 1);
}

csa_status csa_index_topk_paged(const void* q_idx, int q_fmt, const float* w_idx,
                                const void* k_pool, int k_fmt, const csa_block_table* kt,
                                const int32_t* pos, int ratio, int B, int Q, int Hi, int topk,
                                int bf16_scores, int32_t* out_idx, float* out_scores, void* ws,
                                size_t ws_bytes, csa_stream_t stream) {
  PageMap pm;
  csa_status st = page_map(kt, 32, &pm);
  if (st != CSA_OK) return st;
  REQUIRE(bf16_scores == 0 || bf16_scores == 1, CSA_EINVAL, "bf16_scores must be 0 or 1");
  return index_topk(q_idx, q_fmt, w_idx, k_pool, k_fmt, pos, ratio, B, Q, Hi,
                    kt->max_blocks * kt->block_entries, topk, out_idx, out_scores, ws, ws_bytes,
                    stream, bf16_scores, pm);
}

// ---------------------------------------------------------------- attention
static csa_status check_attn(const AttnArgs& a) {
  REQUIRE(a.B >= 1 && a.Q >= 1, CSA_EINVAL, "B and Q must be >= 1");
  REQUIRE(a.ent_seqs >= 1 && a.B % a.ent_seqs == 0, CSA_EINVAL,
          "ent_seqs must divide B (got %d for B = %d)", a.ent_seqs, a.B);
  REQUIRE(a.H >= 16 && a.H % 16 == 0 && a.H <= 1024, CSA_EUNSUPPORTED,
          "H must be a multiple of 16 in [16, 1024]");
  REQUIRE(a.q_fmt == CSA_F32 || a.q_fmt == CSA_BF16, CSA_EUNSUPPORTED, "q_fmt must be F32 or BF16");
  REQUIRE(a.out_fmt == CSA_F32 || a.out_fmt == CSA_BF16, CSA_EUNSUPPORTED, "out_fmt must be F32 or BF16");
  REQUIRE(row_fmt(a.win_fmt) && (row_fmt(a.ent_fmt) || a.ent_fmt == CSA_MIX576), CSA_EUNSUPPORTED,
          "window rows must be F32, BF16, FP8_MX32 or FP4_E4M3_16; entry rows also MIX576");
  REQUIRE(a.ent_fmt != CSA_MIX576 || a.q_fmt == CSA_BF16, CSA_EUNSUPPORTED,
          "MIX576 entry rows need BF16 queries");
  if (a.q_fmt == CSA_BF16)
    REQUIRE(a.win_fmt != CSA_F32 && a.ent_fmt != CSA_F32, CSA_EUNSUPPORTED,
            "F32 rows need F32 queries");
  REQUIRE(a.win_mode == CSA_WIN_RING128 || a.win_mode == CSA_WIN_LINEAR, CSA_EINVAL, "bad win_mode");
  REQUIRE(a.win_rows >= (a.win_mode == CSA_WIN_RING128 ? 128 : 1), CSA_EINVAL,
          "win_rows must be >= 128 in ring mode and >= 1 in linear mode");
  REQUIRE(a.win_rows <= ((int64_t)1 << 31) - 1, CSA_EINVAL, "win_rows too large");
  REQUIRE(a.Nmax >= 0 && a.Nmax <= (int64_t)1 << 30, CSA_EINVAL, "Nmax must be in [0, 2^30]");
  REQUIRE(a.rope_rows >= 1, CSA_EINVAL, "rope_rows must be >= 1");
  REQUIRE(isfinite(a.scale), CSA_EINVAL, "scale must be finite");
  REQUIRE_PTR(a.q);
  REQUIRE_PTR(a.win);
  if (a.Nmax > 0) REQUIRE_PTR(a.entries);
  REQUIRE_PTR(a.pos);
  REQUIRE_PTR(a.sink);
  REQUIRE_PTR(a.rope_cos);
  REQUIRE_PTR(a.rope_sin);
  REQUIRE_PTR(a.out);
  if (a.win_mode == CSA_WIN_LINEAR) REQUIRE_PTR(a.win_base);
  return CSA_OK;
}

size_t csa_sparse_attn_workspace_size(int B, int Q, int H, int topk) {
  if (B < 1 || Q < 1 || H < 16 || topk < 0) return 0;
  AttnArgs a{};
  a.B = B; a.Q = Q; a.H = H; a.topk = topk; a.q_fmt = CSA_BF16; a.dense = 0;
  return attn_ws_bytes(a);
}

size_t hca_attn_workspace_size(int B, int Q, int H, int64_t Nmax) {
  if (B < 1 || Q < 1 || H < 16 || Nmax < 0) return 0;
  AttnArgs a{};
  a.B = B; a.Q = Q; a.H = H; a.Nmax = Nmax; a.q_fmt = CSA_BF16; a.ratio = 128; a.dense = 1;
  const size_t plain = attn_ws_bytes(a);
  // a paged list may be split into more chunks: enough for either call
  static const int32_t kAnyTable = 0;
  a.ent_pages = PageMap{&kAnyTable, 1, 1, 0};
  const size_t paged = attn_ws_bytes(a);
  return plain > paged ? plain : paged;
}

static csa_status run_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  csa_status st = check_attn(a);
  if (st != CSA_OK) return st;
  size_t need = attn_ws_bytes(a);
  REQUIRE(need == 0 || (ws != nullptr && aligned16(ws) && ws_bytes >= need), CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  return launched(launch_attention(a, ws, s), "attention");
}

static AttnArgs make_attn(const void* q, int q_fmt, const void* win, int win_fmt, int win_mode,
                          const int32_t* win_base, int64_t win_rows, const void* entries,
                          int ent_fmt, int64_t Nmax, const int32_t* pos, int B, int Q, int H,
                          const float* sink, float scale, const float* rope_cos,
                          const float* rope_sin, int64_t rope_rows, void* out, int out_fmt) {
  AttnArgs a{};
  a.q = q; a.q_fmt = q_fmt;
  a.win = win; a.win_fmt = win_fmt; a.win_mode = win_mode; a.win_base = win_base;
  a.win_rows = win_rows;
  a.entries = entries; a.ent_fmt = ent_fmt; a.Nmax = Nmax;
  a.pos = pos; a.B = B; a.Q = Q; a.H = H; a.ent_seqs = B;
  a.sink = sink; a.scale = scale;
  a.rope_cos = rope_cos; a.rope_sin = rope_sin; a.rope_rows = rope_rows;
  a.out = out; a.out_fmt = out_fmt;
  return a;
}

csa_status csa_sparse_attn_decode(const void* q, int q_fmt, const void* win, int win_fmt,
                                  int win_mode, const int32_t* win_base, int64_t win_rows,
                                  const void* entries, int ent_fmt, int64_t Nmax,
                                  const int32_t* topk_idx, int topk, const int32_t* pos, int B,
                                  int Q, int H, const float* sink, float scale,
                                  const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                                  void* out, int out_fmt, void* ws, size_t ws_bytes,
                                  csa_stream_t stream) {
  REQUIRE(topk >= 0 && topk <= 8192, CSA_EUNSUPPORTED, "topk must be in [0, 8192]");
  if (topk > 0) REQUIRE_PTR(topk_idx);
  AttnArgs a = make_attn(q, q_fmt, win, win_fmt, win_mode, win_base, win_rows, entries, ent_fmt,
                         Nmax, pos, B, Q, H, sink, scale, rope_cos, rope_sin, rope_rows, out,
                         out_fmt);
  a.dense = 0;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.ratio = 4;
  return run_attn(a, ws, ws_bytes, (hipStream_t)stream);
}

csa_status csa_sparse_attn_decode_shared(const void* q, int q_fmt, const void* win, int win_fmt,
                                         const void* entries, int ent_fmt, int64_t Nmax,
                                         const int32_t* topk_idx, int topk, const int32_t* pos,
                                         int B, int Q, int H, int ent_seqs, const float* sink,
                                         float scale, const float* rope_cos,
                                         const float* rope_sin, int64_t rope_rows, void* out,
                                         int out_fmt, void* ws, size_t ws_bytes,
                                         csa_stream_t stream) {
  REQUIRE(topk >= 0 && topk <= 8192, CSA_EUNSUPPORTED, "topk must be in [0, 8192]");
  REQUIRE(ent_seqs >= 1 && B % ent_seqs == 0, CSA_EINVAL,
          "ent_seqs must divide B (got %d for B = %d)", ent_seqs, B);
  if (topk > 0) REQUIRE_PTR(topk_idx);
  AttnArgs a = make_attn(q, q_fmt, win, win_fmt, CSA_WIN_RING128, nullptr, kWindow, entries,
                         ent_fmt, Nmax, pos, B, Q, H, sink, scale, rope_cos, rope_sin, rope_rows,
                         out, out_fmt);
  a.ent_seqs = ent_seqs;
  a.dense = 0;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.ratio = 4;
  return run_attn(a, ws, ws_bytes, (hipStream_t)stream);
}

csa_status hca_attn_decode(const void* q, int q_fmt, const void* win, int win_fmt, int win_mode,
                           const int32_t* win_base, int64_t win_rows, const void* entries,
                           int ent_fmt, int64_t Nmax, int ratio, const int32_t* pos, int B, int Q,
                           int H, const float* sink, float scale, const float* rope_cos,
                           const float* rope_sin, int64_t rope_rows, void* out, int out_fmt,
                           void* ws, size_t ws_bytes, csa_stream_t stream) {
  REQUIRE(ratio >= 1, CSA_EINVAL, "ratio must be >= 1");
  AttnArgs a = make_attn(q, q_fmt, win, win_fmt, win_mode, win_base, win_rows, entries, ent_fmt,
                         Nmax, pos, B, Q, H, sink, scale, rope_cos, rope_sin, rope_rows, out,
                         out_fmt);
  a.dense = 1;
  a.ratio = ratio;
  return run_attn(a, ws, ws_bytes, (hipStream_t)stream);
}

// Block-cache variants: the contiguous calls with entries through a block
// table and the ring window of sequence b in state slot win_slot[b].
static csa_status paged_attn(AttnArgs& a, const int32_t* win_slot, int64_t win_slots,
                             const csa_block_table* et) {
  csa_status st = page_map(et, 1, &a.ent_pages);
  if (st != CSA_OK) return st;
  REQUIRE(et->pool_blocks * et->block_entries <= INT32_MAX, CSA_EINVAL,
          "an entry pool holds at most 2^31 - 1 rows");
  REQUIRE(win_slots >= 1 && win_slots <= INT32_MAX, CSA_EINVAL, "win_slots must be in [1, 2^31 - 1]");
  REQUIRE(win_slot != nullptr || win_slots >= a.B, CSA_EINVAL,
          "without win_slot the window pool needs win_slots >= B");
  if (win_slot) REQUIRE_PTR(win_slot);
  a.win_slot = win_slot;
  a.win_slots = win_slot ? win_slots : a.B;
  a.Nmax = et->max_blocks * et->block_entries;
  return CSA_OK;
}

csa_status csa_sparse_attn_decode_paged(const void* q, int q_fmt, const void* win_pool,
                                        int win_fmt, const int32_t* win_slot,
                                        int64_t win_slots, const void* ent_pool, int ent_fmt,
                                        const csa_block_table* et, const int32_t* topk_idx,
                                        int topk, const int32_t* pos, int B, int Q, int H,
                                        const float* sink, float scale, const float* rope_cos,
                                        const float* rope_sin, int64_t rope_rows, void* out,
                                        int out_fmt, void* ws, size_t ws_bytes,
                                        csa_stream_t stream) {
  REQUIRE(topk >= 0 && topk <= 8192, CSA_EUNSUPPORTED, "topk must be in [0, 8192]");
  if (topk > 0) REQUIRE_PTR(topk_idx);
  AttnArgs a = make_attn(q, q_fmt, win_pool, win_fmt, CSA_WIN_RING128, nullptr, kWindow,
                         ent_pool, ent_fmt, 0, pos, B, Q, H, sink, scale, rope_cos, rope_sin,
                         rope_rows, out, out_fmt);
  csa_status st = paged_attn(a, win_slot, win_slots, et);
  if (st != CSA_OK) return st;
  a.dense = 0;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.ratio = 4;
  return run_attn(a, ws, ws_bytes, (hipStream_t)stream);
}

csa_status hca_attn_decode_paged(const void* q, int q_fmt, const void* win_pool, int win_fmt,
                                 const int32_t* win_slot, int64_t win_slots,
                                 const void* ent_pool, int ent_fmt, const csa_block_table* et,
                                 int ratio, const int32_t* pos, int B, int Q, int H,
                                 const float* sink, float scale, const float* rope_cos,
                                 const float* rope_sin, int64_t rope_rows, void* out,
                                 int out_fmt, void* ws, size_t ws_bytes, csa_stream_t stream) {
  REQUIRE(ratio >= 1, CSA_EINVAL, "ratio must be >= 1");
  AttnArgs a = make_attn(q, q_fmt, win_pool, win_fmt, CSA_WIN_RING128, nullptr, kWindow,
                         ent_pool, ent_fmt, 0, pos, B, Q, H, sink, scale, rope_cos, rope_sin,
                         rope_rows, out, out_fmt);
  csa_status st = paged_attn(a, win_slot, win_slots, et);
  if (st != CSA_OK) return st;
  a.dense = 1;
  a.ratio = ratio;
  return run_attn(a, ws, ws_bytes, (hipStream_t)stream);
}

// ---------------------------------------------------------------- layer input / output
static csa_status check_layer_shape(const csa_layer_weights* w, int M) {
  REQUIRE(w != nullptr, CSA_EINVAL, "weights must not be null");
  REQUIRE(M >= 1 && M <= 64, CSA_EUNSUPPORTED, "M = B*T must be in [1, 64] (got %d)", M);
  REQUIRE(w->dim >= 256 && w->dim % 256 == 0, CSA_EINVAL, "dim must be a positive multiple of 256");
  REQUIRE(w->q_rank >= 256 && w->q_rank % 256 == 0 && w->q_rank <= 2048, CSA_EINVAL,
          "q_rank must be a multiple of 256 in [256, 2048]");
  REQUIRE(w->H >= 1 && w->H <= 128, CSA_EUNSUPPORTED, "H must be in [1, 128]");
  REQUIRE(w->Hi >= 0 && w->Hi <= 64, CSA_EUNSUPPORTED, "Hi must be in [0, 64]");
  REQUIRE(w->groups >= 1 && w->H % w->groups == 0, CSA_EINVAL, "groups must divide H");
  REQUIRE(w->o_rank >= 32 && w->o_rank % 32 == 0, CSA_EINVAL,
          "o_rank must be a positive multiple of 32");
  REQUIRE(w->eps >= 0 && isfinite(w->eps), CSA_EINVAL, "eps must be finite and >= 0");
  return CSA_OK;
}

size_t csa_layer_input_workspace_size(const csa_layer_weights* w, int M) {
  if (check_layer_shape(w, M) != CSA_OK) return 0;
  return layer_input_ws_bytes(w, M);
}

size_t csa_layer_output_workspace_size(const csa_layer_weights* w, int M) {
  if (check_layer_shape(w, M) != CSA_OK) return 0;
  return layer_output_ws_bytes(w, M);
}

csa_status csa_layer_input(const csa_layer_weights* w, const void* x, const int32_t* pos, int B,
                           int T, const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                           void* q, void* q_idx, float* w_idx, void* win, int win_fmt, void* ws,
                           size_t ws_bytes, csa_stream_t stream) {
  REQUIRE(B >= 1 && T >= 1, CSA_EINVAL, "B and T must be >= 1");
  REQUIRE((int64_t)B * T <= 64, CSA_EUNSUPPORTED, "M = B*T must be in [1, 64]");
  const int M = B * T;
  csa_status st = check_layer_shape(w, M);
  if (st != CSA_OK) return st;
  REQUIRE(row_fmt(win_fmt), CSA_EUNSUPPORTED,
          "win_fmt must be F32, BF16, FP8_MX32 or FP4_E4M3_16");
  REQUIRE(rope_rows >= 1, CSA_EINVAL, "rope_rows must be >= 1");
  REQUIRE_PTR(w->wq_a);
  REQUIRE_PTR(w->q_norm);
  REQUIRE_PTR(w->wq_b);
  REQUIRE_PTR(w->wkv);
  REQUIRE_PTR(w->kv_norm);
  REQUIRE_PTR(x);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(rope_cos);
  REQUIRE_PTR(rope_sin);
  REQUIRE_PTR(q);
  REQUIRE_PTR(win);
  if (w->Hi > 0) {
    REQUIRE_PTR(w->wq_b_idx);
    REQUIRE_PTR(w->w_proj);
    REQUIRE_PTR(q_idx);
    REQUIRE_PTR(w_idx);
  }
  const size_t need = layer_input_ws_bytes(w, M);
  REQUIRE(ws != nullptr && aligned16(ws) && ws_bytes >= need, CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  return launched(launch_layer_input(w, x, pos, B, T, rope_cos, rope_sin, rope_rows, q, q_idx,
                                     w_idx, win, win_fmt, kv_row_bytes(win_fmt, kHeadDim), ws,
                                     (hipStream_t)stream),
                  "csa_layer_input");
}

csa_status csa_layer_output(const csa_layer_weights* w, const void* o, int M, void* y, int y_fmt,
                            void* ws, size_t ws_bytes, csa_stream_t stream) {
  csa_status st = check_layer_shape(w, M);
  if (st != CSA_OK) return st;
  REQUIRE(y_fmt == CSA_F32 || y_fmt == CSA_BF16, CSA_EUNSUPPORTED, "y_fmt must be F32 or BF16");
  REQUIRE_PTR(w->wo_a);
  REQUIRE_PTR(w->wo_b);
  REQUIRE_PTR(o);
  REQUIRE_PTR(y);
  const size_t need = layer_output_ws_bytes(w, M);
  REQUIRE(ws != nullptr && aligned16(ws) && ws_bytes >= need, CSA_EWORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  return launched(launch_layer_output(w, o, M, y, y_fmt, ws, (hipStream_t)stream),
                  "csa_layer_output");
}

}  // extern "C"
