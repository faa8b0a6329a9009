// Internal declarations shared by the host API (api.cpp) and the kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/csa.h"

namespace csa {

constexpr int kWindow = 128;      // raw sliding window rows per query
constexpr int kHeadDim = 512;     // main KV / query head width
constexpr int kIndexDim = 128;    // indexer head width
constexpr int kRopeDims = 64;     // rotated tail of every head
constexpr int kTopkMax = 2048;    // largest k handled by the selection kernels
constexpr int kHistBins = 4096;   // first radix digit: key bits 31..20
constexpr int kCandCap = 8192;    // boundary-bin candidates kept per row

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Block-cache addressing ("DeepSeek-V4 deep dive" section 9.4): logical
// entry e of sequence b is pool row (table[b][e >> shift] << shift) +
// (e & (2^shift - 1)).  table == nullptr selects the contiguous layout, in
// which sequence b's rows start at row b * Nmax.
struct PageMap {
  const int32_t* table;  // [B][max_blocks], or nullptr
  int64_t max_blocks;
  int64_t pool_blocks;
  int shift;             // log2(entries per block)
};

// Sets the calling thread's error detail (csa_last_error_detail) and returns code.
csa_status set_error(csa_status code, const char* fmt, ...);

// ---- launchers (kernel files); each returns hipSuccess or the launch error
hipError_t launch_rope_table(const double* omega_host, int64_t rows, float* cos_out,
                             float* sin_out, hipStream_t s);

hipError_t launch_quantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                           int dim, hipStream_t s);
hipError_t launch_dequantize(const void* src, int src_fmt, void* dst, int dst_fmt, int64_t rows,
                             int dim, hipStream_t s);

// top-k workspace layout for R rows
struct TopkWs {
  uint32_t* hist;    // [R][kHistBins] first digit (key bits 31..20)
  uint32_t* ctr;     // [R][8]: per-row counters and boundary-bin info
  uint32_t* cand;    // [R][kCandCap][2] (key, idx) for the boundary bin
  uint32_t* hi;      // [R][kTopkMax][2] (key, idx) above the boundary bin
};
size_t topk_ws_bytes(int64_t R);
TopkWs topk_ws_carve(void* ws, int64_t R);

hipError_t launch_topk_clear(TopkWs w, int64_t R, hipStream_t s);
hipError_t launch_topk_hist(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld,
                            TopkWs w, hipStream_t s);
hipError_t launch_topk_select(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld,
                              int topk, int32_t* out_idx, TopkWs w, hipStream_t s);

// indexer scores: writes scores[row][s] for s < n_vis and the radix histogram
hipError_t launch_index_scores(const void* q_idx, int q_fmt, const float* w_idx,
                               const void* k_idx, int k_fmt, const int32_t* pos, int ratio, int B,
                               int Q, int Hi, int64_t Nmax, float* scores, int32_t* n_vis,
                               TopkWs w, int bf16_scores, hipStream_t s,
                               PageMap pm = PageMap{nullptr, 0, 0, 0});

struct AttnArgs {
  const void* q; int q_fmt;
  const void* win; int win_fmt; int win_mode; const int32_t* win_base; int64_t win_rows;
  const void* entries; int ent_fmt; int64_t Nmax;
  PageMap ent_pages;                   // entries through a block table (table == nullptr: none)
  const int32_t* win_slot;             // ring window of sequence b is win[win_slot[b]] (nullptr: b)
  int64_t win_slots;                   // slots in the window pool (a slot outside: no window rows)
  int ent_seqs;                        // sequence b reads entry set and top-k list b % ent_seqs
                                       // and sinks [b / ent_seqs][H] (B: one set per sequence)
  int dense;                           // 0: top-k list (CSA), 1: all completed entries (HCA)
  const int32_t* topk_idx; int topk;   // CSA list
  int ratio;                           // HCA visibility ratio
  const int32_t* pos; int B, Q, H;
  const float* sink; float scale;
  const float* rope_cos; const float* rope_sin; int64_t rope_rows;
  void* out; int out_fmt;
  size_t win_rb, ent_rb;               // row bytes (set by the launcher)
  int64_t unit_off;                    // first unit of a sub-grid (set by the launcher)
};
int attn_chunk_rows(const AttnArgs& a);            // rows per work-group chunk
int64_t attn_list_len(const AttnArgs& a);          // max rows in a unit's list
size_t attn_ws_bytes(const AttnArgs& a);
hipError_t launch_attention(const AttnArgs& a, void* ws, hipStream_t s);

size_t compress_ws_bytes(const csa_compress_args* a);
hipError_t launch_compress(const csa_compress_args* a, void* ws, hipStream_t s);
size_t compress_many_ws_bytes(const csa_compress_args* a, int n);
hipError_t launch_compress_many(const csa_compress_args* a, int n, void* ws, hipStream_t s);

size_t layer_input_ws_bytes(const csa_layer_weights* w, int M);
size_t layer_output_ws_bytes(const csa_layer_weights* w, int M);
hipError_t launch_layer_input(const csa_layer_weights* w, const void* x, const int32_t* pos, int B,
                              int T, const float* rope_cos, const float* rope_sin,
                              int64_t rope_rows, void* q, void* q_idx, float* w_idx, void* win,
                              int win_fmt, size_t win_rb, void* ws, hipStream_t s);
hipError_t launch_layer_output(const csa_layer_weights* w, const void* o, int M, void* y,
                               int y_fmt, void* ws, hipStream_t s);

}  // namespace csa
