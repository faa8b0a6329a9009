// Exact, deterministic top-k over float32 scores ("DeepSeek-V4 deep dive"
// section 5.2, step 5: keep min(k, visible blocks) entries).
//
// Order: descending score, equal scores by ascending index, -0 == +0, NaN last.
// Scores map to order-preserving uint32 keys.  A radix select finds the
// threshold key in three digits (12 + 12 + 8 bits):
//   1. a 4096-bin histogram of key >> 20 per row (built by the scoring kernel
//      or by topk_hist_kernel) gives the boundary bin;
//   2. every work-group of the row re-reads its chunk and appends the entries
//      above the boundary bin and those inside it to per-row lists;
//   3. the last work-group of the row to finish refines the boundary bin with
//      the remaining 20 bits, resolves ties at the threshold by index, sorts
//      the winners and writes the row.  If the boundary bin overflows its list
//      the same refinement runs over the whole row instead.
// Counters use integer atomics only, and every list is sorted by a total order
// before it is used, so the result does not depend on scheduling.
#include "common.h"

namespace csa {

namespace {

constexpr int kSelThreads = 256;
constexpr int kChunk = 8192;       // elements scanned per work-group
constexpr int kSortCap = kTopkMax; // winners above the threshold
constexpr int kTieCap = kCandCap;  // equal-to-threshold entries sorted by index

struct RowCtr {
  uint32_t n_hi, n_eq, done, pad;
};

__device__ __forceinline__ bool before(uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Bitonic sort of n (power of two) (key, idx) pairs in LDS, key desc / idx asc.
__device__ void bitonic_pairs(uint32_t* key, uint32_t* idx, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int p = i ^ j;
        if (p > i) {
          bool up = (i & k) == 0;
          uint32_t ki = key[i], kp = key[p], ii = idx[i], ip = idx[p];
          bool swap = up ? before(kp, ip, ki, ii) : before(ki, ii, kp, ip);
          if (swap) { key[i] = kp; key[p] = ki; idx[i] = ip; idx[p] = ii; }
        }
      }
      __syncthreads();
    }
  }
}

// Bitonic sort of n (power of two) uint32 ascending.
__device__ void bitonic_u32(uint32_t* v, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int p = i ^ j;
        if (p > i) {
          bool up = (i & k) == 0;
          uint32_t a = v[i], b = v[p];
          if (up ? (b < a) : (a < b)) { v[i] = b; v[p] = a; }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Find the largest bin b with sum_{b' >= b} hist[b'] >= need (need >= 1 and the
// total >= need).  hist lives in LDS, nbins is a multiple of kSelThreads.
// Returns b and writes the count strictly above b to *above.  Ends synced.
__device__ int suffix_find(const uint32_t* hist, int nbins, uint32_t need, uint32_t* above,
                           uint32_t* scratch /* LDS, kSelThreads + 2 */) {
  const int per = nbins / kSelThreads;
  const int t = threadIdx.x;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += hist[t * per + j];
  scratch[t] = local;
  __syncthreads();
  if (t == 0) {
    // serial suffix over thread totals (256 adds), then within the owner
    uint32_t acc = 0;
    int owner = 0;
    for (int u = kSelThreads - 1; u >= 0; --u) {
      if (acc + scratch[u] >= need) { owner = u; break; }
      acc += scratch[u];
    }
    int b = owner * per;
    for (int j = per - 1; j >= 0; --j) {
      uint32_t h = hist[owner * per + j];
      if (acc + h >= need) { b = owner * per + j; break; }
      acc += h;
    }
    scratch[kSelThreads] = (uint32_t)b;
    scratch[kSelThreads + 1] = acc;
  }
  __syncthreads();
  int b = (int)scratch[kSelThreads];
  *above = scratch[kSelThreads + 1];
  __syncthreads();
  return b;
}

struct LdsSel {
  uint32_t hist[kHistBins];
  uint32_t scratch[kSelThreads + 8];
  uint32_t skey[kSortCap];
  uint32_t sidx[kSortCap];
  uint32_t ties[kTieCap];
  uint32_t n_sel, n_ties, flag;
};

// Source of (key, idx) pairs for the refinement: either the boundary-bin list
// of a row (unordered) or the whole row of scores (index order).
struct ListSrc {
  const uint32_t* pairs;  // [n][2]
  uint32_t n;
  __device__ uint32_t size() const { return n; }
  __device__ void get(uint32_t i, uint32_t& k, uint32_t& ix) const {
    k = pairs[2 * i];
    ix = pairs[2 * i + 1];
  }
};
struct RowSrc {
  const float* s;
  uint32_t n;
  __device__ uint32_t size() const { return n; }
  __device__ void get(uint32_t i, uint32_t& k, uint32_t& ix) const {
    k = score_key(s[i]);
    ix = i;
  }
};

// Refine the boundary bin b1 (key >> 20) of a row, collect every element of the
// bin with key > T plus the `need`-rank ties, and append them to L.skey/L.sidx
// (after the n_pre elements already there) / L.ties.  ordered: the source is in
// ascending index order (ties are then taken in scan order without sorting).
template <class Src>
__device__ void refine_and_collect(const Src& src, uint32_t b1, uint32_t need, bool ordered,
                                   LdsSel& L) {
  const int t = threadIdx.x;
  const uint32_t n = src.size();
  // digit 2: bits 19..8 within b1
  for (int i = t; i < kHistBins; i += kSelThreads) L.hist[i] = 0;
  __syncthreads();
  for (uint32_t i = t; i < n; i += kSelThreads) {
    uint32_t k, ix;
    src.get(i, k, ix);
    if ((k >> 20) == b1) atomicAdd(&L.hist[(k >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  uint32_t above2;
  uint32_t b2 = (uint32_t)suffix_find(L.hist, kHistBins, need, &above2, L.scratch);
  // digit 3: bits 7..0 within (b1, b2)
  const uint32_t pre = (b1 << 12) | b2;
  for (int i = t; i < kHistBins; i += kSelThreads) L.hist[i] = 0;
  __syncthreads();
  for (uint32_t i = t; i < n; i += kSelThreads) {
    uint32_t k, ix;
    src.get(i, k, ix);
    if ((k >> 8) == pre) atomicAdd(&L.hist[k & 0xffu], 1u);
  }
  __syncthreads();
  uint32_t above3;
  // 256 bins: pad the rest of the histogram with zeros (already zero)
  uint32_t b3 = (uint32_t)suffix_find(L.hist, kHistBins, need - above2, &above3, L.scratch);
  const uint32_t T = (pre << 8) | b3;
  const uint32_t need_t = need - above2 - above3;  // >= 1 ties to take at key T
  // collect key > T within the bin (count above2 + above3 < need <= kSortCap)
  for (uint32_t i = t; i < n; i += kSelThreads) {
    uint32_t k, ix;
    src.get(i, k, ix);
    if ((k >> 20) == b1 && k > T) {
      uint32_t slot = atomicAdd(&L.n_sel, 1u);
      if (slot < (uint32_t)kSortCap) {
        L.skey[slot] = k;
        L.sidx[slot] = ix;
      }
    }
  }
  __syncthreads();
  if (!ordered) {
    // all ties into L.ties (the boundary list holds at most kTieCap entries)
    for (uint32_t i = t; i < n; i += kSelThreads) {
      uint32_t k, ix;
      src.get(i, k, ix);
      if (k == T) {
        uint32_t slot = atomicAdd(&L.n_ties, 1u);
        if (slot < (uint32_t)kTieCap) L.ties[slot] = ix;
      }
    }
    __syncthreads();
    int m = (int)L.n_ties < kTieCap ? (int)L.n_ties : kTieCap;
    int p2 = pow2_at_least(m);
    for (int i = m + t; i < p2; i += kSelThreads) L.ties[i] = 0xffffffffu;
    __syncthreads();
    bitonic_u32(L.ties, p2);
    if (t == 0) L.n_ties = need_t;
    __syncthreads();
  } else {
    // take the first need_t ties in index order, one block of the row at a time
    if (t == 0) L.n_ties = 0;
    __syncthreads();
    for (uint32_t base = 0; base < n; base += kSelThreads) {
      uint32_t i = base + t;
      bool f = false;
      uint32_t k = 0, ix = 0;
      if (i < n) {
        src.get(i, k, ix);
        f = (k == T);
      }
      // block-wide exclusive prefix of the flags
      unsigned long long bal = __ballot(f);
      int lane = t & 63, wv = t >> 6;
      uint32_t pre_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) L.scratch[wv] = __popcll(bal);
      __syncthreads();
      uint32_t off = 0;
      for (int u = 0; u < wv; ++u) off += L.scratch[u];
      uint32_t tot = L.scratch[0] + L.scratch[1] + L.scratch[2] + L.scratch[3];
      uint32_t have = L.n_ties;
      if (f && have + off + pre_in_wave < need_t) L.ties[have + off + pre_in_wave] = ix;
      __syncthreads();
      if (t == 0) L.n_ties = have + tot;
      __syncthreads();
      if (L.n_ties >= need_t) break;
    }
    if (t == 0) L.n_ties = need_t;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kSelThreads) topk_clear_kernel(uint32_t* hist, uint32_t* ctr,
                                                                  int64_t R) {
  int64_t n = R * kHistBins;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    hist[i] = 0;
    if (i < R * 4) ctr[i] = 0;
  }
}

__global__ void __launch_bounds__(kSelThreads) topk_hist_kernel(const float* __restrict__ scores,
                                                                 const int32_t* __restrict__ n_valid,
                                                                 int64_t ld, uint32_t* hist) {
  __shared__ uint32_t h[kHistBins];
  const int64_t row = blockIdx.y;
  int64_t nv = n_valid[row];
  nv = nv < 0 ? 0 : (nv > ld ? ld : nv);
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  if (base >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) h[i] = 0;
  __syncthreads();
  const float* s = scores + row * ld;
  int64_t end = base + kChunk < nv ? base + kChunk : nv;
  for (int64_t i = base + threadIdx.x; i < end; i += kSelThreads)
    atomicAdd(&h[score_key(s[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = hist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_valid, int64_t ld, int topk,
    int32_t* __restrict__ out_idx, const uint32_t* hist_g, RowCtr* ctr_g, uint32_t* cand_g,
    uint32_t* hi_g) {
  __shared__ LdsSel L;
  const int t = threadIdx.x;
  const int64_t row = blockIdx.y;
  int64_t nv64 = n_valid[row];
  nv64 = nv64 < 0 ? 0 : (nv64 > ld ? ld : nv64);
  const uint32_t nv = (uint32_t)nv64;
  const uint32_t k_eff = nv < (uint32_t)topk ? nv : (uint32_t)topk;
  const uint32_t nchunks = (nv + kChunk - 1) / kChunk;
  RowCtr* ctr = ctr_g + row;
  uint32_t* cand = cand_g + row * (int64_t)kCandCap * 2;
  uint32_t* hi = hi_g + row * (int64_t)kTopkMax * 2;
  int32_t* out = out_idx + row * (int64_t)topk;
  const float* s = scores + row * ld;

  if (k_eff == 0) {  // nothing visible: one work-group pads the row
    if (blockIdx.x == 0)
      for (int i = t; i < topk; i += kSelThreads) out[i] = -1;
    return;
  }
  if (blockIdx.x >= nchunks) return;

  // boundary bin from the row histogram
  for (int i = t; i < kHistBins; i += kSelThreads) L.hist[i] = hist_g[row * kHistBins + i];
  __syncthreads();
  uint32_t above;
  const uint32_t b1 = (uint32_t)suffix_find(L.hist, kHistBins, k_eff, &above, L.scratch);
  const uint32_t eq = L.hist[b1];
  const bool keep_eq = eq <= (uint32_t)kCandCap;

  // append this chunk's entries above / inside the boundary bin
  const uint32_t base = blockIdx.x * (uint32_t)kChunk;
  const uint32_t end = base + kChunk < nv ? base + kChunk : nv;
  for (uint32_t i = base + t; i < end; i += kSelThreads) {
    uint32_t k = score_key(s[i]);
    uint32_t b = k >> 20;
    if (b > b1) {
      uint32_t slot = atomicAdd(&ctr->n_hi, 1u);
      if (slot < (uint32_t)kTopkMax) {  // always true: fewer than k_eff lie above b1
        hi[2 * slot] = k;
        hi[2 * slot + 1] = i;
      }
    } else if (b == b1 && keep_eq) {
      uint32_t slot = atomicAdd(&ctr->n_eq, 1u);
      if (slot < (uint32_t)kCandCap) {  // always true: eq <= kCandCap
        cand[2 * slot] = k;
        cand[2 * slot + 1] = i;
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (t == 0) L.flag = (atomicAdd(&ctr->done, 1u) == nchunks - 1) ? 1u : 0u;
  __syncthreads();
  if (!L.flag) return;
  __threadfence();

  // ---- last work-group of the row: finish the selection
  if (t == 0) { L.n_sel = 0; L.n_ties = 0; }
  __syncthreads();
  // entries above the boundary bin (fewer than k_eff)
  for (uint32_t i = t; i < above && i < (uint32_t)kSortCap; i += kSelThreads) {
    L.skey[i] = hi[2 * i];
    L.sidx[i] = hi[2 * i + 1];
  }
  if (t == 0) L.n_sel = above;
  __syncthreads();
  const uint32_t need = k_eff - above;
  if (keep_eq) {
    ListSrc src{cand, eq};
    refine_and_collect(src, b1, need, false, L);
  } else {
    RowSrc src{s, nv};
    refine_and_collect(src, b1, need, true, L);
  }
  // sort the winners above the threshold, then append the ties in index order
  const int n_sel = (int)L.n_sel < kSortCap ? (int)L.n_sel : kSortCap;
  const int p2 = pow2_at_least(n_sel < 1 ? 1 : n_sel);
  for (int i = n_sel + t; i < p2; i += kSelThreads) { L.skey[i] = 0u; L.sidx[i] = 0xffffffffu; }
  __syncthreads();
  bitonic_pairs(L.skey, L.sidx, p2);
  for (int i = t; i < topk; i += kSelThreads) {
    int32_t v = -1;
    if (i < n_sel) v = (int32_t)L.sidx[i];
    else if ((uint32_t)i < k_eff) v = (int32_t)L.ties[i - n_sel];
    out[i] = v;
  }
}

}  // namespace

size_t topk_ws_bytes(int64_t R) {
  size_t b = align_up((size_t)R * kHistBins * 4, 256);
  b += align_up((size_t)R * 16, 256);
  b += align_up((size_t)R * kCandCap * 8, 256);
  b += align_up((size_t)R * kTopkMax * 8, 256);
  return b;
}

TopkWs topk_ws_carve(void* ws, int64_t R) {
  char* p = (char*)ws;
  TopkWs w;
  w.hist = (uint32_t*)p;
  p += align_up((size_t)R * kHistBins * 4, 256);
  w.ctr = (uint32_t*)p;
  p += align_up((size_t)R * 16, 256);
  w.cand = (uint32_t*)p;
  p += align_up((size_t)R * kCandCap * 8, 256);
  w.hi = (uint32_t*)p;
  return w;
}

hipError_t launch_topk_clear(TopkWs w, int64_t R, hipStream_t s) {
  int64_t n = R * kHistBins;
  int64_t blocks = (n + kSelThreads - 1) / kSelThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0, s, w.hist,
                     w.ctr, R);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld,
                            TopkWs w, hipStream_t s) {
  int64_t gx = (ld + kChunk - 1) / kChunk;
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)gx, (unsigned)nr), dim3(kSelThreads), 0, s,
                       scores + r0 * ld, n_valid + r0, ld, w.hist + r0 * kHistBins);
  }
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, const int32_t* n_valid, int64_t R, int64_t ld,
                              int topk, int32_t* out_idx, TopkWs w, hipStream_t s) {
  int64_t gx = (ld + kChunk - 1) / kChunk;
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)gx, (unsigned)nr), dim3(kSelThreads), 0,
                       s, scores + r0 * ld, n_valid + r0, ld, topk, out_idx + r0 * topk,
                       w.hist + r0 * kHistBins, (RowCtr*)w.ctr + r0,
                       w.cand + r0 * (int64_t)kCandCap * 2, w.hi + r0 * (int64_t)kTopkMax * 2);
  }
  return hipGetLastError();
}

}  // namespace csa
