/*
 * libcsa -- DeepSeek-V4-style compressed-attention decode for one layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one described in "DeepSeek-V4 deep dive" (gangliao.me):
 *   - a learned gated-pooling compressor turns every m = 4 (CSA) or m = 128
 *     (HCA) tokens into one 512-d entry that is both key and value for all
 *     query heads (sections 3.1, 4.1-4.3);
 *   - a lightning indexer scores every completed entry with 128-d index heads
 *     and keeps the top k (section 5.2);
 *   - shared-KV multi-query attention runs one softmax with a per-head sink over
 *     the raw 128-token window plus the selected entries, with RoPE on the last
 *     64 dims undone on the output (sections 3.3, 3.4 Eq. 27, 5.3, 6.1).
 * Cache row formats follow the V4-Flash model record (528 B FP8 rows, 288 B
 * FP4 rows) and the V4.1-Flash diagram page (E2M1 + E4M3 scale per 16).
 * Around the path: the layer's query path, index-query preparation and
 * window-entry write (csa_layer_input) and its grouped low-rank output
 * projection (csa_layer_output), sections 3.2, 3.5 and 5.2; the V4.1 CSA2
 * compressor at m = 2 and m = 1 and layer groups that share main KV and top-k
 * ids (csa_sparse_attn_decode_shared), V4.1-Flash diagram page.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library never allocates or frees and keeps no state between
 *     calls.  Scratch memory is passed in as a workspace sized by the matching
 *     *_workspace_size() call.
 *   - Tensors are dense, row-major, last dimension contiguous, and must start
 *     on a 16-byte boundary.
 *   - Work is enqueued on `stream`; calls return without synchronising.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation failure nothing is written, the return value is non-zero and
 *     csa_last_error_detail() describes the problem.  A failed launch returns
 *     CSA_ELAUNCH.  Nothing throws across this interface.  Calls are
 *     thread-safe; the error detail is per thread.
 *   - Values stored in device memory cannot be checked on the host.  Position
 *     arrays and index lists are clamped or masked by the kernels as stated per
 *     function; they never cause an out-of-bounds access.
 *   - Results are bitwise reproducible run to run and batch-invariant: the
 *     output for one sequence does not depend on the batch it is part of.
 *     Kernels are chosen by the shape of a call per sequence, never by the
 *     batch: with 12 or more queries per sequence (bf16 index keys) the
 *     indexer scores tiles of queries together, bit-identically to one-query
 *     calls; with 16 or more queries per sequence the sparse attention takes
 *     640-row chunks (64 heads: all heads per work-group), which may round
 *     differently from the 64-row chunks of fewer queries.
 *   - Positions are absolute token positions (0-based).  Compressed entry ids
 *     are 0-based in compressed space; -1 means "no row".
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* csa_stream_t; /* a hipStream_t; NULL = default stream */
typedef int csa_status;

enum {
  CSA_OK = 0,
  CSA_EINVAL = 1,       /* bad argument (null pointer, size, alignment)        */
  CSA_EUNSUPPORTED = 2, /* valid but unsupported combination of formats/shapes */
  CSA_EWORKSPACE = 3,   /* workspace missing or smaller than required          */
  CSA_ELAUNCH = 4       /* a kernel launch failed                              */
};

/* Storage formats of a row of `dim` values. */
enum {
  CSA_F32 = 0,          /* 4*dim bytes                                                   */
  CSA_BF16 = 1,         /* 2*dim bytes                                                   */
  CSA_FP8_MX32 = 2,     /* dim OCP-E4M3FN codes, then dim/32 E8M0 scale bytes (e + 127):
                           528 B for dim 512, 132 B for dim 128                          */
  CSA_FP4_E4M3_16 = 3,  /* dim/2 bytes of E2M1 codes (element 2j in the low nibble of
                           byte j), then dim/16 E4M3 scale bytes: 288 B for dim 512      */
  CSA_FP4_MX32 = 4,     /* OCP MX FP4 ("DeepSeek-V4 deep dive" section 5.2 notes: the
                           FP4 indexer): dim/2 bytes of E2M1 codes (element 2j in the low
                           nibble of byte j), then dim/32 E8M0 scale bytes X + 127 with
                           X = floor(log2 amax) - 2 clamped to [-127, 127] (amax 0 ->
                           -127); codes RNE(x / 2^X) saturating at 6; a non-finite group
                           gets scale 0xFF and zero codes.  68 B per 128-d index key.
                           Index keys and kv_quantize / kv_dequantize only.            */
  CSA_MIX576 = 5        /* the V4 mixed row ("DeepSeek-V4 deep dive" sections 3.1, 3.3
                           notes: 448 FP8 + 64 bf16 = 576 bytes before scales, FP8 in
                           blocks of 64), dim 512 only: 448 E4M3 codes (the FP8_MX32 rule
                           per block of 64), the 64 RoPE dims as bf16 (RNE), 7 E8M0
                           scale bytes, 9 zero bytes: 592 B.  Codec, compressor entries
                           and attention entry rows.                                    */
};

/* Addressing of the raw sliding-window rows. */
enum {
  CSA_WIN_RING128 = 0,  /* decode: the row of position p is p mod 128 of a 128-row ring  */
  CSA_WIN_LINEAR = 1    /* prefill: the row of position p is p - win_base[b]             */
};

const char* csa_strerror(csa_status s);
/* Text of the last failure on the calling thread ("" when none). */
const char* csa_last_error_detail(void);
/* Bytes per row of `dim` values in `fmt`; 0 if the pair is invalid. */
size_t kv_row_bytes(int fmt, int dim);

/* ------------------------------------------------------------------------ RoPE
 * cos/sin table for the partial RoPE of "DeepSeek-V4 deep dive" section 3.3 and
 * the YaRN settings of section 9.1.  Pair k (dims D-64+2k, D-64+2k+1 of a row)
 * turns by angle p * omega_k with omega_k = theta^(-2k/64); when yarn_factor > 0
 * the frequencies are blended as omega' = omega/factor*(1-s) + omega*s with
 * s = 1 - clamp((k-lo)/(hi-lo), 0, 1) and (lo, hi) the YaRN correction range
 * of (beta_fast, beta_slow) over yarn_orig_len positions.  The angle is
 * formed in double precision and cos/sin are rounded once to float.
 * Writes cos_out[rows][32] and sin_out[rows][32] (device) for positions
 * 0 .. rows-1.  Errors: CSA_EINVAL for null outputs, rows < 1, theta <= 1.   */
csa_status csa_rope_table(double theta, double yarn_factor, int64_t yarn_orig_len,
                          double beta_fast, double beta_slow, int64_t rows, float* cos_out,
                          float* sin_out, csa_stream_t stream);

/* ------------------------------------------------------------------------ codec
 * Storage rounding of cache rows (the FP8 / FP4 row layouts of the V4-Flash
 * model record; V4.1 page: E2M1 with an E4M3 scale per 16 channels).
 * kv_quantize: src [rows][dim] in CSA_F32 or CSA_BF16 -> dst rows in dst_fmt
 *   (any format).  FP8_MX32: per 32 values the scale is 2^e with e the smallest
 *   integer such that max|x| <= 448 * 2^e (clamped to [-127,127]; all-zero
 *   groups use -127); codes are x * 2^-e rounded to nearest even E4M3FN,
 *   saturating at +-448.  FP4_E4M3_16: per 16 values scale = E4M3(RNE(max|x| /
 *   6)) in IEEE float32, codes = RNE onto the E2M1 grid of x / scale, ties to
 *   the even code, saturating at 6; a zero scale gives zero codes.  NaN or Inf
 *   inputs become NaN codes (FP8) or a NaN scale (FP4) so that they propagate.
 * kv_dequantize: src rows in src_fmt -> dst [rows][dim] in CSA_F32 or CSA_BF16
 *   (bf16 rounds to nearest even).
 * dim must be a positive multiple of 32 (of 128 for FP8_MX32, whose rows must
 * stay 4-byte aligned).  rows may be 0 (no work).                           */
csa_status kv_quantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                       int dim, csa_stream_t stream);
csa_status kv_dequantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                         int dim, csa_stream_t stream);

/* ------------------------------------------------------------------------ compressor
 * "DeepSeek-V4 deep dive" sections 4.1-4.3 and 5.2.  For each token at
 * position p = start_pos[b] + i (i < T) of sequence b:
 *   v = W_kv x,  s = W_gate x + ape[p mod ratio]          (each coff*head_dim wide)
 * The projections are written into the caller's slot state (layout below).
 * Whenever a block completes ((p+1) mod ratio == 0) entry p/ratio is emitted:
 *   ratio 4 (overlap, coff 2): 8 slots = previous block's tokens on channels
 *     [0, d) followed by the current block's tokens on channels [d, 2d);
 *   ratio 128 (coff 1): the block's 128 tokens;  ratio 2 (coff 1): the
 *     block's 2 tokens, without overlap (the CSA2 compressor of the
 *     V4.1-Flash diagram page at m = 2; its missing slot bias is a zero ape);
 *   ratio 1: the single token (CSA2 at m = 1);
 *   C_c = sum_j softmax_j(s_{j,c}) v_{j,c}  per channel, in float32;
 *   y = C / sqrt(mean(C^2) + eps) * norm_w;  RoPE on the last 64 dims at
 *   position (p/ratio)*ratio;  if rotate: y = H y / sqrt(head_dim) with H the
 *   Sylvester Hadamard matrix (head_dim 128 index keys only);  then storage
 *   rounding to entry_fmt, written to entries[b][p/ratio] (skipped when
 *   p/ratio >= entries_cap).
 * Slot state (in/out, float32, [B][coff*ratio][coff*head_dim] each): the slot
 * of position p is ratio + p mod ratio when coff == 2, else p mod ratio.  On a
 * completed block with coff == 2 the current slots are copied into the
 * previous slots [0, ratio).  A fresh state is kv = 0 and score = -inf.
 * Positions before start_pos[b] are taken from the state as it holds them.
 * x: [B][T][dim] in x_fmt (F32 or BF16); w_kv, w_gate: [coff*head_dim][dim] in
 * w_fmt (F32 or BF16); ape: [ratio][coff*head_dim] float; norm_w: [head_dim]
 * float; rope tables [rope_rows][32] float (positions beyond rope_rows - 1 are
 * clamped to the last row); start_pos: [B] int32.
 * Requirements: ratio in {1, 2, 4, 128}; head_dim in {128, 512}; rotate only with
 * head_dim 128; dim % 32 == 0; entry_fmt any; B >= 1, T >= 1.            */
typedef struct {
  int B, T, dim, ratio, head_dim, rotate;
  const void* x;
  int x_fmt;
  const void* w_kv;
  const void* w_gate;
  int w_fmt;
  const float* ape;
  const float* norm_w;
  float eps;
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_rows;
  const int32_t* start_pos;
  float* kv_state;
  float* score_state;
  void* entries;
  int entry_fmt;
  int64_t entries_cap;
  /* Block cache (optional; all zero = the contiguous layout above; see
   * csa_block_table below).  When block_table is set, `entries` is a pool of
   * pool_blocks blocks of block_entries rows, entry i of sequence b is
   * written to row i mod block_entries of block block_table[b][i /
   * block_entries], and entries_cap is replaced by max_blocks *
   * block_entries; an entry whose block id is -1 or outside [0, pool_blocks)
   * is not written.  When state_slot is set, kv_state and score_state are
   * pools of state_slots slots and sequence b uses slot state_slot[b]; a
   * sequence whose slot lies outside [0, state_slots) is skipped (nothing
   * read or written for it).  Two sequences of one call must not share a
   * slot (the caller's guarantee). */
  const int32_t* block_table;
  int64_t max_blocks;
  int block_entries;
  int64_t pool_blocks;
  const int32_t* state_slot;
  int64_t state_slots;
} csa_compress_args;

size_t csa_compress_workspace_size(const csa_compress_args* a);
csa_status csa_compress(const csa_compress_args* a, void* ws, size_t ws_bytes,
                        csa_stream_t stream);

/* Several compressors in one call (the same section: a CSA layer runs its
 * 512-wide main-KV compressor and its 128-wide index-key compressor on the
 * same token).  The result equals calling csa_compress on a[0], ..., a[n-1]
 * in order; the calls must not share state or entries buffers.  When every
 * call is single-token (T == 1) with bf16 x and weights, dim % 256 == 0 and
 * the same B <= 1024, their projections run as one launch and their emits as
 * another.  A sequence's entries and slot state do not depend on B.
 * n in [1, 4].  Workspace: csa_compress_many_workspace_size(a, n) bytes
 * (16-byte aligned); errors as for csa_compress, reported for the first
 * failing call before anything is enqueued.                             */
size_t csa_compress_many_workspace_size(const csa_compress_args* a, int n);
csa_status csa_compress_many(const csa_compress_args* a, int n, void* ws, size_t ws_bytes,
                             csa_stream_t stream);

/* ------------------------------------------------------------------------ indexer + top-k
 * "DeepSeek-V4 deep dive" section 5.2:  for query (b, q) at position
 * pos[b][q] the visible blocks are s < n_vis = min(floor((pos+1)/ratio), Nmax);
 *   score[s] = sum_h w[b][q][h] * max(0, q_idx[b][q][h] . k[b][s])
 * computed with float32 accumulation (bf16 products are exact in float32;
 * FP8 keys are decoded exactly), then the top min(topk, n_vis) entries are
 * returned in out_idx[b][q][0..topk) ordered by descending score, equal scores
 * by ascending index, -0 == +0, NaN last; the remaining slots hold -1.
 * q_idx: [B][Q][Hi][128] in q_fmt (F32 or BF16), or [B][Q][Hi] rows of 68 B
 * in q_fmt FP4_MX32 (the key codec's MXFP4 rows); w_idx: [B][Q][Hi] float,
 * with the 128^-1/2 * Hi^-1/2 factor already applied; k_idx: [B][Nmax] rows of
 * 128 values in k_fmt (F32, BF16, FP8_MX32 = 132 B or FP4_MX32 = 68 B);
 * pos: [B][Q] int32.
 * out_scores (nullable): [B][Q][Nmax] float, entries s < n_vis are written.
 * Requirements: Hi % 16 == 0 and Hi <= 128 (any Hi for F32); 1 <= topk <= 2048;
 * k_fmt F32 requires q_fmt F32, BF16/FP8 require q_fmt BF16, and FP4_MX32
 * keys take q_fmt BF16 or FP4_MX32.  With FP4_MX32 queries and keys a 16 x 16
 * block of head-key products is one block-scaled FP4 MFMA over all 128 dims
 * (E2M1 products are exact; float32 accumulation).                          */
size_t csa_index_topk_workspace_size(int B, int Q, int64_t Nmax, int topk);
csa_status csa_index_topk(const void* q_idx, int q_fmt, const float* w_idx, const void* k_idx,
                          int k_fmt, const int32_t* pos, int ratio, int B, int Q, int Hi,
                          int64_t Nmax, int topk, int32_t* out_idx, float* out_scores, void* ws,
                          size_t ws_bytes, csa_stream_t stream);

/* The FP4 indexer's scoring ("DeepSeek-V4 deep dive" section 5.2 notes: FP4
 * index keys and queries after the Hadamard rotation, BF16 index scores):
 * exactly csa_index_topk, except that every score is rounded to bf16
 * (round to nearest even; NaN stays NaN) before it is stored in out_scores and
 * ranked.  Ties that the rounding creates are broken by the smaller index, as
 * in csa_index_topk.  Meant for k_fmt = CSA_FP4_MX32 keys (68 B per key) with
 * FP4_MX32 queries (or bf16 queries that carry FP4 values: an E2M1 code times
 * a power of two is exact in bf16); any k_fmt that csa_index_topk accepts is
 * accepted.  Same arguments, workspace size and errors.                      */
csa_status csa_index_topk_bf16(const void* q_idx, int q_fmt, const float* w_idx,
                               const void* k_idx, int k_fmt, const int32_t* pos, int ratio,
                               int B, int Q, int Hi, int64_t Nmax, int topk, int32_t* out_idx,
                               float* out_scores, void* ws, size_t ws_bytes,
                               csa_stream_t stream);

/* csa_index_topk for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and errors without the workspace.  Its scratch is a
 * fixed 32 MiB array inside the library, one per device, held until the
 * process ends; csa_index_topk_workspace_size(B, Q, Nmax, topk) must not
 * exceed 32 MiB (8 sequences of 262,144 entries need 9.2 MB), else the call
 * returns CSA_EWORKSPACE before enqueuing anything.  The call makes no
 * allocation of any kind.  Its first call on a device resolves that device's
 * scratch address (hipGetSymbolAddress), so make one call before capturing a
 * graph.  Every call on a device shares that device's scratch: calls that
 * overlap on one device (different streams, or different threads) race and
 * must be serialised by the caller.  The scratch keeps the last call's
 * contents; the call clears what it needs itself.                          */
csa_status csa_index_topk_noalloc(const void* q_idx, int q_fmt, const float* w_idx,
                                  const void* k_idx, int k_fmt, const int32_t* pos, int ratio,
                                  int B, int Q, int Hi, int64_t Nmax, int topk, int32_t* out_idx,
                                  float* out_scores, csa_stream_t stream);

/* Top-k alone over given float32 scores [R][ld]: row r ranks its first
 * n_valid[r] entries (clamped to [0, ld]) with the same order rule as above.
 * Requirements: 1 <= topk <= 2048, ld >= 1.                                  */
size_t csa_topk_workspace_size(int64_t R, int64_t ld, int topk);
csa_status csa_topk(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld, int topk,
                    int32_t* out_idx, void* ws, size_t ws_bytes, csa_stream_t stream);

/* ------------------------------------------------------------------------ attention
 * Shared-KV MQA with a sink ("DeepSeek-V4 deep dive" section 3.4, Eq. 27) over
 * the list [128 window rows ; selected entries] of each query unit (b, q):
 *   window row j (0..127) is position t-127+j with t = pos[b][q]; it is absent
 *   when that position is negative, else read from win[b] at row
 *   (position mod 128) in CSA_WIN_RING128 mode or (position - win_base[b]) in
 *   CSA_WIN_LINEAR mode (absent when outside [0, win_rows));
 *   csa_sparse_attn_decode: entry rows topk_idx[b][q][0..topk), -1 or any id
 *   outside [0, Nmax) is absent;
 *   hca_attn_decode: entry rows 0 .. min(floor((t+1)/ratio), Nmax) - 1.
 * Per head h, with q' = RoPE(q[b][q][h], t) on the last 64 dims and rows c_j
 * in stored (already rotated) form:
 *   z_j = (q' . c_j) * scale,  m = max_j z_j,
 *   o = sum_j e^{z_j - m} c_j / (sum_j e^{z_j - m} + e^{sink[h] - m}),
 *   out = RoPE^-1(o, t) on the last 64 dims   (duplicates are kept);
 * no present row gives out = 0.  Products use bf16 MFMA with float32
 * accumulation (the softmax weights are rounded to bf16 for the second
 * product) except for q_fmt F32, which runs in float32 throughout.
 * q: [B][Q][H][512] in q_fmt (F32 or BF16), passed UN-rotated; win: [B][win_rows]
 * rows of 512 in win_fmt; entries: [B][Nmax] rows of 512 in ent_fmt; formats
 * F32 (only with q_fmt F32), BF16, FP8_MX32, FP4_E4M3_16; sink: [H] float;
 * rope tables [rope_rows][32] (positions clamped to the last row); out:
 * [B][Q][H][512] in out_fmt (F32 or BF16, rounded once).
 * Batch invariance ("DeepSeek-V4 deep dive" section 10.5, the systems box's
 * batch-invariant decode attention): a unit's output depends only on its own
 * inputs, never on B or on the other units.  The
 * library combines a list's fixed 64-row chunks in chunk order whether one
 * work-group takes the whole list (large batches) or each chunk has its own
 * work-group (small batches); the workspace, which holds the chunks' partial
 * results in the second case, may be empty (size 0) in the first.
 * Requirements: H % 16 == 0; win_rows >= 128 in ring mode; 0 <= topk <= 8192.
 */
size_t csa_sparse_attn_workspace_size(int B, int Q, int H, int topk);
csa_status csa_sparse_attn_decode(const void* q, int q_fmt, const void* win, int win_fmt,
                                  int win_mode, const int32_t* win_base, int64_t win_rows,
                                  const void* entries, int ent_fmt, int64_t Nmax,
                                  const int32_t* topk_idx, int topk, const int32_t* pos, int B,
                                  int Q, int H, const float* sink, float scale,
                                  const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                                  void* out, int out_fmt, void* ws, size_t ws_bytes,
                                  csa_stream_t stream);

/* Layers that share main KV and top-k ids (the CSA2 layer groups of the
 * V4.1-Flash diagram page: a Full layer and its Reuse layers).  The same as
 * csa_sparse_attn_decode with a decode ring window (CSA_WIN_RING128), for B
 * sequences that form B / ent_seqs groups of ent_seqs: sequence b attends with
 * its own q[b], window win[b] and output out[b], reads entry set
 * entries[b % ent_seqs] through the top-k list topk_idx[b % ent_seqs], and
 * takes its sinks from sink[b / ent_seqs][H].  Laid out as layer-major
 * groups: b = layer * ent_seqs + s.  One launch serves every layer.
 * entries: [ent_seqs][Nmax][row]; topk_idx: [ent_seqs][Q][topk]; q, out:
 * [B][Q][H][512]; win: [B][128][row]; pos: [B][Q]; sink: [B / ent_seqs][H].
 * Workspace: csa_sparse_attn_workspace_size(B, Q, H, topk).  Errors as for
 * csa_sparse_attn_decode, and CSA_EINVAL unless ent_seqs divides B.         */
csa_status csa_sparse_attn_decode_shared(const void* q, int q_fmt, const void* win, int win_fmt,
                                         const void* entries, int ent_fmt, int64_t Nmax,
                                         const int32_t* topk_idx, int topk, const int32_t* pos,
                                         int B, int Q, int H, int ent_seqs, const float* sink,
                                         float scale, const float* rope_cos,
                                         const float* rope_sin, int64_t rope_rows, void* out,
                                         int out_fmt, void* ws, size_t ws_bytes,
                                         csa_stream_t stream);

size_t hca_attn_workspace_size(int B, int Q, int H, int64_t Nmax);
csa_status hca_attn_decode(const void* q, int q_fmt, const void* win, int win_fmt, int win_mode,
                           const int32_t* win_base, int64_t win_rows, const void* entries,
                           int ent_fmt, int64_t Nmax, int ratio, const int32_t* pos, int B, int Q,
                           int H, const float* sink, float scale, const float* rope_cos,
                           const float* rope_sin, int64_t rope_rows, void* out, int out_fmt,
                           void* ws, size_t ws_bytes, csa_stream_t stream);

/* ------------------------------------------------------------------------ block cache
 * The serving layout of "DeepSeek-V4 deep dive" section 9.4: compressed
 * entries (and, for CSA, their index keys) live in a pool of fixed-size
 * blocks, each covering a multiple of 128 tokens -- 32 CSA entries or 1 HCA
 * entry per 128 tokens -- found through a per-sequence block table; what is
 * still in motion (the 128-row window ring and the compressors' slot state)
 * lives in one fixed-size state slot per request, drawn from a pool.
 * Logical entry e of sequence b is row e mod block_entries of pool block
 * table[b][e / block_entries]; the logical capacity is Nmax = max_blocks *
 * block_entries.  A pool is [pool_blocks][block_entries][row bytes].
 * The paged calls compute exactly what their contiguous counterparts compute
 * on the gathered rows, in the same order: their results are bit-identical
 * to the contiguous calls' on the same logical data.                      */
typedef struct {
  const int32_t* table;   /* [B][max_blocks] int32 (device): the pool block of each
                             logical block of each sequence; -1 = not allocated   */
  int64_t max_blocks;     /* length of a table row, >= 1                           */
  int block_entries;      /* entries per block: a power of two in [1, 1024]; index
                             keys need >= 32 (one 128-token CSA block)             */
  int64_t pool_blocks;    /* blocks in the pool, >= 1                              */
} csa_block_table;

/* csa_index_topk (bf16_scores = 0) or csa_index_topk_bf16 (bf16_scores = 1)
 * over index keys held in a block pool: k_pool [pool_blocks][block_entries]
 * rows of 128 values in k_fmt, found through kt (kt->block_entries >= 32).
 * Nmax = kt->max_blocks * kt->block_entries; out_idx holds logical entry ids,
 * out_scores (nullable) is [B][Q][Nmax].  A visible key whose block id is -1
 * or outside [0, pool_blocks) is read as a zero key (score 0); nothing
 * outside the pool is read.  Workspace: csa_index_topk_workspace_size(B, Q,
 * Nmax, topk).  Errors as for csa_index_topk, and CSA_EINVAL for a bad
 * table descriptor.  With 12 or more bf16-key queries per sequence the scan
 * runs the per-query kernel (bit-identical to the query-tiled one).        */
csa_status csa_index_topk_paged(const void* q_idx, int q_fmt, const float* w_idx,
                                const void* k_pool, int k_fmt, const csa_block_table* kt,
                                const int32_t* pos, int ratio, int B, int Q, int Hi, int topk,
                                int bf16_scores, int32_t* out_idx, float* out_scores, void* ws,
                                size_t ws_bytes, csa_stream_t stream);

/* csa_sparse_attn_decode (ring window) and hca_attn_decode over a block pool
 * and state slots: sequence b's 128-row window ring is win_pool[win_slot[b]]
 * (win_pool: [win_slots][128] rows; win_slot NULL means slot b, and then
 * win_slots must be >= B), and its entries are ent_pool rows found through
 * et (Nmax = et->max_blocks * et->block_entries).  A slot outside
 * [0, win_slots) leaves the sequence without window rows.  A list id (CSA)
 * or visible entry (HCA) whose block id is -1 or outside [0, pool_blocks) is
 * absent, like an id outside [0, Nmax).  Entry pools hold at most 2^31 - 1
 * rows (pool_blocks * block_entries).
 * Workspace: csa_sparse_attn_workspace_size(B, Q, H, topk) and
 * hca_attn_workspace_size(B, Q, H, Nmax) (sized for either HCA call).  Errors as for the contiguous
 * calls, and CSA_EINVAL for a bad table descriptor.                       */
csa_status csa_sparse_attn_decode_paged(const void* q, int q_fmt, const void* win_pool,
                                        int win_fmt, const int32_t* win_slot,
                                        int64_t win_slots, const void* ent_pool, int ent_fmt,
                                        const csa_block_table* et, const int32_t* topk_idx,
                                        int topk, const int32_t* pos, int B, int Q, int H,
                                        const float* sink, float scale, const float* rope_cos,
                                        const float* rope_sin, int64_t rope_rows, void* out,
                                        int out_fmt, void* ws, size_t ws_bytes,
                                        csa_stream_t stream);
csa_status hca_attn_decode_paged(const void* q, int q_fmt, const void* win_pool, int win_fmt,
                                 const int32_t* win_slot, int64_t win_slots,
                                 const void* ent_pool, int ent_fmt,
                                 const csa_block_table* et, int ratio, const int32_t* pos, int B,
                                 int Q, int H, const float* sink, float scale,
                                 const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                                 void* out, int out_fmt, void* ws, size_t ws_bytes,
                                 csa_stream_t stream);

/* ------------------------------------------------------------------------ layer input / output
 * The attention layer's steps on either side of the decode path, for M = B*T
 * tokens (T per sequence, row m = b*T + i at position pos[m]).
 *
 * csa_layer_input ("DeepSeek-V4 deep dive" sections 3.2, 3.3, 3.4 notes, 5.2):
 *   qr = RMSNorm(wq_a x) * q_norm, rounded to bf16 (the shared query latent);
 *   q[m][h]  = v_h / sqrt(mean(v_h^2) + eps),  v = wq_b qr split into H heads
 *              of 512 (the per-head rescale has no weight).  q is written
 *              UN-rotated: the page's query is RoPE_p(q[m][h]), and the
 *              attention calls (csa_sparse_attn_decode, hca_attn_decode) take
 *              exactly this un-rotated q and rotate it at the query position
 *              themselves, so the output feeds them directly;
 *   kv       = RoPE_p(RMSNorm(wkv x) * kv_norm), stored in win_fmt into row
 *              p mod 128 of sequence b's window ring win[b][128][row]
 *              (skipped for p < 0);
 *   when Hi > 0 (CSA layers):
 *   q_idx[m][h] = H128 RoPE_p(u_h) / sqrt(128),  u = wq_b_idx qr split into Hi
 *              heads of 128, H128 the Sylvester Hadamard matrix;
 *   w_idx[m][h] = (w_proj x)_h / sqrt(128 * Hi).
 *   RMSNorm(v) = v / sqrt(mean(v^2) + eps); RoPE_p rotates the last 64 dims at
 *   position p as csa_rope_table describes (p clamped to [0, rope_rows-1]).
 *   x: [M][dim] bf16.  Outputs: q [M][H][512] bf16, q_idx [M][Hi][128] bf16,
 *   w_idx [M][Hi] float (both unused when Hi == 0), win in win_fmt (F32, BF16,
 *   FP8_MX32 or FP4_E4M3_16 rows of 512).
 * csa_layer_output (section 3.5, grouped low-rank output projection):
 *   the H heads of o form `groups` groups of H/groups consecutive heads;
 *   mid[m][g*o_rank + r] = sum_d o[m][g][d] wo_a[g][r][d]   (rounded to bf16)
 *   y[m][n] = sum_j mid[m][j] wo_b[n][j],  y in y_fmt (F32 or BF16).
 *   o: [M][H][512] bf16 (the attention output, RoPE already undone).
 * Weights (device, bf16 unless noted; row-major [out][in]):
 *   wq_a [q_rank][dim]; q_norm [q_rank] float; wq_b [H*512][q_rank];
 *   wkv [512][dim]; kv_norm [512] float; wq_b_idx [Hi*128][q_rank];
 *   w_proj [Hi][dim]; wo_a [groups][o_rank][H/groups*512]; wo_b [dim][groups*o_rank].
 *   Pointers a call does not use may be NULL (the output weights for
 *   csa_layer_input, the input weights for csa_layer_output, the index
 *   weights when Hi == 0).
 * Products use bf16 operands with float32 accumulation; the K split of each
 * product depends on the weight shapes only, so results do not depend on B.
 * Requirements: 1 <= M <= 64; dim a positive multiple of 256; q_rank a
 * multiple of 256 in [256, 2048];
 * 1 <= H <= 128; 0 <= Hi <= 64; groups >= 1 with H % groups == 0; o_rank a
 * positive multiple of 32; eps finite and >= 0.  Workspaces: the matching
 * *_workspace_size(w, M) bytes, 16-byte aligned.  Errors: CSA_EINVAL for null
 * or misaligned pointers and bad sizes, CSA_EUNSUPPORTED for formats,
 * CSA_EWORKSPACE for a short workspace.                                        */
typedef struct {
  int dim, q_rank, H, Hi, groups, o_rank;
  const void* wq_a;
  const float* q_norm;
  const void* wq_b;
  const void* wkv;
  const float* kv_norm;
  const void* wq_b_idx;
  const void* w_proj;
  const void* wo_a;
  const void* wo_b;
  float eps;
} csa_layer_weights;

size_t csa_layer_input_workspace_size(const csa_layer_weights* w, int M);
csa_status csa_layer_input(const csa_layer_weights* w, const void* x, const int32_t* pos, int B,
                           int T, const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                           void* q, void* q_idx, float* w_idx, void* win, int win_fmt, void* ws,
                           size_t ws_bytes, csa_stream_t stream);
size_t csa_layer_output_workspace_size(const csa_layer_weights* w, int M);
csa_status csa_layer_output(const csa_layer_weights* w, const void* o, int M, void* y, int y_fmt,
                            void* ws, size_t ws_bytes, csa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
