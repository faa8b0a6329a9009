// Exact, deterministic top-k over float32 scores ("DeepSeek-V4 deep dive"
// section 5.2, step 5: keep min(k, visible blocks) entries).
//
// Order: descending score, equal scores by ascending index, -0 == +0, NaN last.
// Scores map to order-preserving uint32 keys.  A radix select finds the
// threshold key in three digits (12 + 12 + 8 bits):
//   1. a 4096-bin histogram of key >> 20 per row (built by the scoring kernel
//      or by topk_hist_kernel) gives the boundary bin;
//   2. collect: every work-group re-reads its chunk of the row, finds the
//      boundary bin from the histogram and appends the entries above it and
//      those inside it to per-row lists (positions from one 64-bit atomic per
//      work-group);
//   3. final: one work-group per row refines the boundary bin with the
//      remaining 20 bits, resolves ties at the threshold by index, sorts the
//      winners and writes the row.  If the boundary bin overflowed its list
//      the same refinement runs over the whole row instead.
// The lists are gathered in scheduling order, but every one is reduced to a
// total order (key, then index) before it is used, so the result does not
// depend on scheduling.

#include "common.h"

namespace csa {

namespace {

constexpr int kSelThreads = 256;
constexpr int kChunk = 8192;       // elements scanned per work-group
constexpr int kSortCap = kTopkMax; // winners above the threshold
constexpr int kTieCap = kCandCap;  // equal-to-threshold entries sorted by index


__device__ __forceinline__ bool before(uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
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
// total >= need) over the kHistBins bins of hist (LDS).  Returns b and writes
// the count strictly above b to *above.  Every thread holds 16 consecutive
// bins in registers; a wave prefix sum (suffix = wave total - exclusive
// prefix) plus the higher waves' totals gives each thread the count at and
// above its bins, and the single thread whose range crosses `need` resolves
// the bin from its registers.  Ends synced.
__device__ int suffix_find(const uint32_t* hist, uint32_t need, uint32_t* above,
                           uint32_t* scratch /* LDS, kSelThreads + 8 */) {
  constexpr int per = kHistBins / kSelThreads;
  static_assert(per == 16, "16 bins per thread");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t h[per];
#pragma unroll
  for (int q = 0; q < per / 4; ++q) {
    const uint4 v = *(const uint4*)(hist + per * t + 4 * q);
    h[4 * q] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) local += h[j];
  const uint32_t incl = wave_prefix_incl(local);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if (lane == 0) scratch[w] = total;
  __syncthreads();
  uint32_t S = total - incl + local;  // this thread's bins and the wave's higher ones
  for (int u = w + 1; u < kSelThreads / 64; ++u) S += scratch[u];
  const uint32_t prev = S - local;
  if (S >= need && prev < need) {
    uint32_t acc = prev;
    int b = per * t;
    bool found = false;
#pragma unroll
    for (int j = per - 1; j >= 0; --j) {
      const bool hit = !found && acc + h[j] >= need;
      if (hit) b = per * t + j;
      if (!found && !hit) acc += h[j];
      found = found || hit;
    }
    scratch[kSelThreads] = (uint32_t)b;
    scratch[kSelThreads + 1] = acc;
  }
  __syncthreads();
  const int b = (int)scratch[kSelThreads];
  *above = scratch[kSelThreads + 1];
  __syncthreads();
  return b;
}

// Sort n pairs (n <= kSortCap) by (key desc, idx asc) and write the indices to
// out[0, n).  The pair is packed as key << 32 | ~idx, so one descending 64-bit
// bitonic network over the next power of two orders both keys at once.
__device__ void sort_store(const uint32_t* key, const uint32_t* idx, int n, uint64_t* tmp,
                           int32_t* out) {
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  for (int i = threadIdx.x; i < p2; i += blockDim.x)
    tmp[i] = i < n ? (((uint64_t)key[i] << 32) | (uint64_t)(~idx[i])) : 0ull;
  __syncthreads();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < p2 / 2; i += blockDim.x) {
        const int lo = (i / j) * 2 * j + (i % j), hi = lo + j;
        const bool desc = (lo & k) == 0;
        const uint64_t a = tmp[lo], b = tmp[hi];
        if (desc ? (a < b) : (a > b)) { tmp[lo] = b; tmp[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) out[i] = (int32_t)(~(uint32_t)tmp[i]);
}

struct __align__(16) LdsSel {  // hist is read as 16-byte vectors
  uint32_t hist[kHistBins];
  uint32_t scratch[kSelThreads + 16];
  uint32_t skey[kSortCap];
  uint32_t sidx[kSortCap];
  uint32_t ties[kTieCap];          // also the 64-bit sort buffer (kTieCap / 2 >= kSortCap)
  uint32_t n_sel, n_ties, flag;
};
static_assert(kTieCap / 2 >= kSortCap, "sort buffer");

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
  uint32_t b2 = (uint32_t)suffix_find(L.hist, need, &above2, L.scratch);
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
  uint32_t b3 = (uint32_t)suffix_find(L.hist, need - above2, &above3, L.scratch);
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
    if (i < R * 8) ctr[i] = 0;
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

constexpr int kCandPerThread = kCandCap / kSelThreads;   // 32
constexpr int kHiPerThread = kTopkMax / kSelThreads;      // 8

// Descending sort of 512 packed values held two per lane (element
// e = 128 wave + 2 lane + i).  Bitonic network: partners within a lane or a
// wave are exchanged with register moves and cross-lane shuffles; only the
// stages whose partner lives in another wave go through LDS (3 of 45).
__device__ void sort512_desc(uint64_t (&v)[2], uint64_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = 128 * wave + 2 * lane;
  for (int k = 2; k <= 512; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j == 1) {
        const bool desc = (e0 & k) == 0;
        if (desc ? (v[0] < v[1]) : (v[0] > v[1])) { const uint64_t x = v[0]; v[0] = v[1]; v[1] = x; }
      } else if (j < 128) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t lo = __shfl_xor((uint32_t)v[i], j >> 1, 64);
          const uint32_t hi = __shfl_xor((uint32_t)(v[i] >> 32), j >> 1, 64);
          const uint64_t pv = ((uint64_t)hi << 32) | lo;
          const int e = e0 + i;
          const bool keep_max = ((e & j) == 0) == ((e & k) == 0);
          v[i] = keep_max ? (v[i] > pv ? v[i] : pv) : (v[i] < pv ? v[i] : pv);
        }
      } else {
        __syncthreads();
        lds[e0] = v[0];
        lds[e0 + 1] = v[1];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int e = e0 + i;
          const uint64_t pv = lds[e ^ j];
          const bool keep_max = ((e & j) == 0) == ((e & k) == 0);
          v[i] = keep_max ? (v[i] > pv ? v[i] : pv) : (v[i] < pv ? v[i] : pv);
        }
      }
    }
  }
}

// Lane exchange lane <-> lane ^ M within a wave, for a compile-time M: quad
// permutes (1, 2) and a row rotate (8) on the DPP path, swizzles (4, 16),
// a permute through LDS only for 32.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true);
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true);
  else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, true);
  else if constexpr (M == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (4 << 10));
  else if constexpr (M == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (16 << 10));
  else return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ M) << 2), (int)x);
}

// Bitonic network over 512 packed values held by the four waves of a
// work-group, 2 per lane (element e = 2 (64 wave + lane) + i), sorted
// descending.  Stage (K, J) compares e with e ^ J: inside a lane for J = 1,
// across lanes (lane ^ J/2) for 2 <= J <= 64, across waves through LDS for
// J = 128 and 256.  Lane distances 16 and 32 use the gfx950 row swaps, which
// hand both members of a pair both values, so each keeps the larger or the
// smaller one directly.  Called by all threads of the work-group.
template <int K, int J>
__device__ __forceinline__ void bitonic_stage2(uint64_t (&v)[2], int e0, uint64_t* lds) {
  if constexpr (J == 1) {
    const bool desc = (e0 & K) == 0;
    const uint64_t a = v[0], b = v[1];
    const bool swap = desc ? (a < b) : (a > b);
    v[0] = swap ? b : a;
    v[1] = swap ? a : b;
  } else if constexpr (J == 32 || J == 64) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t alo = (uint32_t)v[i], blo = alo, ahi = (uint32_t)(v[i] >> 32), bhi = ahi;
      if constexpr (J == 32) { swap_rows16(alo, blo); swap_rows16(ahi, bhi); }
      else { swap_halves32(alo, blo); swap_halves32(ahi, bhi); }
      const uint64_t a = ((uint64_t)ahi << 32) | alo, b = ((uint64_t)bhi << 32) | blo;
      const int e = e0 + i;
      const bool keep_max = ((e & J) == 0) == ((e & K) == 0);
      v[i] = keep_max == (a > b) ? a : b;
    }
  } else {
    uint64_t pv[2];
    if constexpr (J < 128) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t lo = lane_xor<J / 2>((uint32_t)v[i]);
        const uint32_t hi = lane_xor<J / 2>((uint32_t)(v[i] >> 32));
        pv[i] = ((uint64_t)hi << 32) | lo;
      }
    } else {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) lds[e0 + i] = v[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) pv[i] = lds[(e0 + i) ^ J];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = e0 + i;
      const bool keep_max = ((e & J) == 0) == ((e & K) == 0);
      v[i] = keep_max ? (v[i] > pv[i] ? v[i] : pv[i]) : (v[i] < pv[i] ? v[i] : pv[i]);
    }
  }
}
template <int K, int J> struct Bitonic2J {
  static __device__ __forceinline__ void run(uint64_t (&v)[2], int e0, uint64_t* lds) {
    bitonic_stage2<K, J>(v, e0, lds);
    Bitonic2J<K, J / 2>::run(v, e0, lds);
  }
};
template <int K> struct Bitonic2J<K, 0> {
  static __device__ __forceinline__ void run(uint64_t (&)[2], int, uint64_t*) {}
};
template <int K> struct Bitonic2K {
  static __device__ __forceinline__ void run(uint64_t (&v)[2], int e0, uint64_t* lds) {
    Bitonic2J<K, K / 2>::run(v, e0, lds);
    Bitonic2K<2 * K>::run(v, e0, lds);
  }
};
template <> struct Bitonic2K<1024> {
  static __device__ __forceinline__ void run(uint64_t (&)[2], int, uint64_t*) {}
};

// lds: 512 uint64
__device__ __forceinline__ void sort512_wg_desc(uint64_t (&v)[2], uint64_t* lds) {
  Bitonic2K<2>::run(v, 2 * (int)threadIdx.x, lds);
}

// Write the indices of n <= kSortCap (key, idx) pairs ordered by key desc,
// idx asc (pairs packed as key << 32 | ~idx).
__device__ void order_store(const uint32_t* key, const uint32_t* idx, int n, uint64_t* tmp,
                            int32_t* out) {
  if (n <= 512) {
    const int e0 = 128 * (threadIdx.x >> 6) + 2 * (threadIdx.x & 63);
    uint64_t v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = e0 + i;
      v[i] = e < n ? (((uint64_t)key[e] << 32) | (uint64_t)(~idx[e])) : 0ull;
    }
    sort512_desc(v, tmp);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (e0 + i < n) out[e0 + i] = (int32_t)(~(uint32_t)v[i]);
    return;
  }
  sort_store(key, idx, n, tmp, out);
}

struct RowInfo {       // written by work-group 0 of each row's collect pass
  unsigned long long counts;  // n_hi | n_eq << 32 (atomic)
  uint32_t b1, above, eq, pad;
};

// Pass 1, every chunk of every row: the first digit's boundary bin from the
// row histogram, then this chunk's entries above the bin go to the row's hi
// list and those inside it to the candidate list.  Each thread keeps its keys
// in registers, a block-wide prefix gives every entry its slot, and one
// 64-bit atomic per work-group reserves its ranges in both lists.  CH
// scores per work-group (8192, or fewer when the rows are few and short, so
// that the pass still spreads over the CUs).
template <int CH>
__global__ void __launch_bounds__(kSelThreads) topk_collect_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_valid, int64_t ld, int topk,
    const uint32_t* hist_g, RowInfo* info_g, uint32_t* cand_g, uint32_t* hi_g) {
  __shared__ __align__(16) uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[kSelThreads + 16];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.y;
  int64_t nv64 = n_valid[row];
  nv64 = nv64 < 0 ? 0 : (nv64 > ld ? ld : nv64);
  const uint32_t nv = (uint32_t)nv64;
  const uint32_t k_eff = nv < (uint32_t)topk ? nv : (uint32_t)topk;
  const uint32_t nchunks = (nv + CH - 1) / CH;
  if (k_eff == 0 || blockIdx.x >= nchunks) return;
  RowInfo* info = info_g + row;
  uint32_t* cand = cand_g + row * (int64_t)kCandCap * 2;
  uint32_t* hi = hi_g + row * (int64_t)kTopkMax * 2;
  const float* s = scores + row * ld;

  const uint32_t base = blockIdx.x * (uint32_t)CH;
  const uint32_t end = base + CH < nv ? base + CH : nv;
  constexpr int kPer = CH / kSelThreads;
  // element of (thread t, slot j): base + 4 (t + 256 (j / 4)) + j % 4, read as
  // float4 (scores first: their latency overlaps the histogram's)
  uint32_t kk[kPer];
  const bool full = base + CH <= nv && (ld & 3) == 0;
  if (full) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const float4 v = *(const float4*)(s + base + 4 * (t + kSelThreads * q));
      kk[4 * q] = score_key(v.x); kk[4 * q + 1] = score_key(v.y);
      kk[4 * q + 2] = score_key(v.z); kk[4 * q + 3] = score_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = base + 4 * (t + kSelThreads * (j >> 2)) + (j & 3);
      kk[j] = i < end ? score_key(s[i]) : 0u;
    }
  }
  {
    uint4 hv[kHistBins / kSelThreads / 4];
#pragma unroll
    for (int q = 0; q < kHistBins / kSelThreads / 4; ++q)
      hv[q] = *(const uint4*)(hist_g + row * kHistBins + 4 * (t + kSelThreads * q));
#pragma unroll
    for (int q = 0; q < kHistBins / kSelThreads / 4; ++q)
      *(uint4*)(hist + 4 * (t + kSelThreads * q)) = hv[q];
  }
  __syncthreads();
  uint32_t above;
  const uint32_t b1 = (uint32_t)suffix_find(hist, k_eff, &above, scratch);
  const uint32_t eq = hist[b1];
  const bool keep_eq = eq <= (uint32_t)kCandCap;
  if (blockIdx.x == 0 && t == 0) {
    info->b1 = b1;
    info->above = above;
    info->eq = eq;
  }
  uint32_t n_hi_t = 0, n_eq_t = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = base + 4 * (t + kSelThreads * (j >> 2)) + (j & 3);
    const uint32_t b = kk[j] >> 20;
    if (i < end && b > b1) ++n_hi_t;
    if (i < end && b == b1) ++n_eq_t;
  }
  const int lane = t & 63, wv = t >> 6;
  // both counts in one prefix sum (a wave's totals stay below 2^16)
  const uint32_t pk = wave_prefix_incl(n_hi_t | (n_eq_t << 16));
  const uint32_t ph = pk & 0xffffu, pe = pk >> 16;
  if (lane == 63) { scratch[wv] = ph; scratch[4 + wv] = pe; }
  __syncthreads();
  uint32_t off_h = ph - n_hi_t, off_e = pe - n_eq_t;
  for (int u = 0; u < wv; ++u) { off_h += scratch[u]; off_e += scratch[4 + u]; }
  if (t == 0) {
    const uint32_t th = scratch[0] + scratch[1] + scratch[2] + scratch[3];
    const uint32_t te = keep_eq ? scratch[4] + scratch[5] + scratch[6] + scratch[7] : 0u;
    const unsigned long long old =
        (th | te) ? atomicAdd(&info->counts, (unsigned long long)th | ((unsigned long long)te << 32))
                  : 0ull;
    scratch[8] = (uint32_t)old;
    scratch[9] = (uint32_t)(old >> 32);
  }
  __syncthreads();
  uint32_t sh = scratch[8] + off_h, se = scratch[9] + off_e;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = base + 4 * (t + kSelThreads * (j >> 2)) + (j & 3);
    if (i >= end) continue;
    const uint32_t b = kk[j] >> 20;
    if (b > b1) {
      if (sh < (uint32_t)kTopkMax) {  // always true: fewer than k_eff lie above b1
        hi[2 * sh] = kk[j];
        hi[2 * sh + 1] = i;
      }
      ++sh;
    } else if (b == b1 && keep_eq) {
      if (se < (uint32_t)kCandCap) {  // always true: eq <= kCandCap
        cand[2 * se] = kk[j];
        cand[2 * se + 1] = i;
      }
      ++se;
    }
  }
}

// Boundary lists of 513..1024 entries: sort entries [0, 512) (already in fv,
// two per lane) and [512, eq) separately with the 512-entry network, keep both
// in LDS, and write the first `need` entries of their descending merge: output
// i takes A[a] or B[i - a], where the co-rank a (entries of A among the first
// i outputs) is the smallest a with A[a] < B[i - a - 1] (packed values are
// distinct: they carry the index).
__device__ void boundary_two_halves(uint64_t (&fv)[2], const uint32_t* cand, uint32_t eq,
                                    uint32_t need, int e0, LdsSel& L, int32_t* out) {
  uint64_t* A = (uint64_t*)L.skey;  // skey and sidx together hold 1024 packed values
  uint64_t* Bh = A + 512;
  sort512_wg_desc(fv, (uint64_t*)L.ties);
  A[e0] = fv[0];
  A[e0 + 1] = fv[1];
  const uint2* src = (const uint2*)cand + 512 + e0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint2 pr = src[i];  // the candidate list always holds these pairs
    fv[i] = (uint32_t)(512 + e0 + i) < eq ? (((uint64_t)pr.x << 32) | (uint64_t)(~pr.y)) : 0ull;
  }
  __syncthreads();  // the first sort's last reads of the buffer are done
  sort512_wg_desc(fv, (uint64_t*)L.ties);
  Bh[e0] = fv[0];
  Bh[e0 + 1] = fv[1];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = e0 + r;
    if ((uint32_t)i >= need) continue;
    int lo = i > 512 ? i - 512 : 0, hi = i < 512 ? i : 512;
    while (lo < hi) {  // first a with !(A[a] > B[i - a - 1])
      const int mid = (lo + hi) >> 1;
      if (A[mid] > Bh[i - mid - 1]) lo = mid + 1;
      else hi = mid;
    }
    const int b = i - lo;
    const uint64_t va = lo < 512 ? A[lo] : 0ull, vb = b < 512 ? Bh[b] : 0ull;
    out[i] = (int32_t)(~(uint32_t)(va > vb ? va : vb));
  }
}

// Pass 2, two work-groups per row.  In the common case (the hi list and the
// boundary list both fit 512 entries and the boundary bin was kept) the first
// work-group orders the hi list and the second the boundary list, each
// writing its part of the row.  Otherwise the first work-group alone refines
// the boundary bin with the remaining 20 bits (12 + 8) from the
// register-resident candidates, resolves ties at the threshold by index,
// orders the winners and writes the row; when the boundary bin held more
// entries than the candidate list, the refinement runs over the whole row.
__global__ void __launch_bounds__(kSelThreads) topk_final_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_valid, int64_t ld, int topk,
    int32_t* __restrict__ out_idx, const RowInfo* info_g, const uint32_t* cand_g,
    const uint32_t* hi_g) {
  __shared__ LdsSel L;
  const int t = threadIdx.x;
  const int part = blockIdx.x;  // 0: hi list (and the general path), 1: boundary list
  const int64_t row = blockIdx.y;
  int64_t nv64 = n_valid[row];
  nv64 = nv64 < 0 ? 0 : (nv64 > ld ? ld : nv64);
  const uint32_t nv = (uint32_t)nv64;
  const uint32_t k_eff = nv < (uint32_t)topk ? nv : (uint32_t)topk;
  int32_t* out = out_idx + row * (int64_t)topk;
  if (k_eff == 0) {
    if (part == 0)
      for (int i = t; i < topk; i += kSelThreads) out[i] = -1;
    return;
  }
  const RowInfo* info = info_g + row;
  const uint32_t* cand = cand_g + row * (int64_t)kCandCap * 2;
  const uint32_t* hi = hi_g + row * (int64_t)kTopkMax * 2;
  const float* s = scores + row * ld;
  // This part's list's first 512 pairs are read before the lengths are known
  // (the workspace always holds them), 2 per lane.
  const int e0 = 2 * t;
  uint64_t fv[2];
  {
    const uint2* src = (const uint2*)(part == 0 ? hi : cand) + e0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint2 pr = src[i];
      fv[i] = ((uint64_t)pr.x << 32) | (uint64_t)(~pr.y);
    }
  }
  const uint32_t b1 = info->b1, above = info->above, eq = info->eq;
  const bool keep_eq = eq <= (uint32_t)kCandCap;
  const uint32_t need = k_eff - above;
  // Fast path: every entry of the hi list outranks every entry of the
  // boundary bin, so the answer is the sorted hi list followed by the first
  // `need` entries of the sorted boundary list.  A boundary list of up to
  // 1024 entries is sorted as two halves whose first `need` (<= 512) merged
  // entries are taken.
  const bool two_halves = eq > 512u && eq <= 1024u && need <= 512u;
  if (keep_eq && above <= 512u && (eq <= 512u || two_halves)) {
    if (part == 1 && two_halves) {
      boundary_two_halves(fv, cand, eq, need, e0, L, out + above);
      for (int i = (int)k_eff + t; i < topk; i += kSelThreads) out[i] = -1;
      return;
    }
    const uint32_t n = part == 0 ? above : eq;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if ((uint32_t)(e0 + i) >= n) fv[i] = 0ull;  // padding sorts last
    sort512_wg_desc(fv, (uint64_t*)L.ties);
    const uint32_t lim = part == 0 ? above : need;
    int32_t* o = out + (part == 0 ? 0u : above);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if ((uint32_t)(e0 + i) < lim) o[e0 + i] = (int32_t)(~(uint32_t)fv[i]);
    if (part == 1)
      for (int i = (int)k_eff + t; i < topk; i += kSelThreads) out[i] = -1;
    return;
  }
  if (part != 0) return;
  if (t == 0) { L.n_sel = 0; L.n_ties = 0; }
  uint32_t hk[kHiPerThread], hx[kHiPerThread];
#pragma unroll
  for (int j = 0; j < kHiPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    hk[j] = i < above ? hi[2 * i] : 0u;
    hx[j] = i < above ? hi[2 * i + 1] : 0u;
  }
  if (!keep_eq) {
#pragma unroll
    for (int j = 0; j < kHiPerThread; ++j) {
      const uint32_t i = t + j * kSelThreads;
      if (i < above) { L.skey[i] = hk[j]; L.sidx[i] = hx[j]; }
    }
    if (t == 0) L.n_sel = above;
    __syncthreads();
    RowSrc src{s, nv};
    refine_and_collect(src, b1, need, true, L);
    const int n_sel = (int)L.n_sel < kSortCap ? (int)L.n_sel : kSortCap;
    // ties (already in index order) follow the ordered winners
    for (int i = t; i < topk; i += kSelThreads)
      if (i >= n_sel) out[i] = (uint32_t)i < k_eff ? (int32_t)L.ties[i - n_sel] : -1;
    __syncthreads();  // L.ties is reused as the sort buffer
    order_store(L.skey, L.sidx, n_sel, (uint64_t*)L.ties, out);
    return;
  }
  uint32_t ck[kCandPerThread], cx[kCandPerThread];
#pragma unroll
  for (int j = 0; j < kCandPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    ck[j] = i < eq ? cand[2 * i] : 0u;
    cx[j] = i < eq ? cand[2 * i + 1] : 0u;
  }
  // second digit: bits 19..8 within b1
  for (int i = t; i < kHistBins; i += kSelThreads) L.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCandPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    if (i < eq) atomicAdd(&L.hist[(ck[j] >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  uint32_t above2;
  const uint32_t b2 = (uint32_t)suffix_find(L.hist, need, &above2, L.scratch);
  const uint32_t pre = (b1 << 12) | b2;
  // third digit: bits 7..0 within (b1, b2)
  for (int i = t; i < kHistBins; i += kSelThreads) L.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCandPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    if (i < eq && (ck[j] >> 8) == pre) atomicAdd(&L.hist[ck[j] & 0xffu], 1u);
  }
  __syncthreads();
  uint32_t above3;
  const uint32_t b3 = (uint32_t)suffix_find(L.hist, need - above2, &above3, L.scratch);
  const uint32_t T = (pre << 8) | b3;
  const uint32_t need_t = need - above2 - above3;  // >= 1 entries equal to T are taken
  // winners: the hi list, candidates above T, and ties at T (by index)
#pragma unroll
  for (int j = 0; j < kHiPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    if (i < above) { L.skey[i] = hk[j]; L.sidx[i] = hx[j]; }
  }
  if (t == 0) L.n_sel = above;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCandPerThread; ++j) {
    const uint32_t i = t + j * kSelThreads;
    if (i < eq) {
      if (ck[j] > T) {
        const uint32_t slot = atomicAdd(&L.n_sel, 1u);
        if (slot < (uint32_t)kSortCap) { L.skey[slot] = ck[j]; L.sidx[slot] = cx[j]; }
      } else if (ck[j] == T) {
        const uint32_t slot = atomicAdd(&L.n_ties, 1u);
        if (slot < (uint32_t)kTieCap) L.ties[slot] = cx[j];
      }
    }
  }
  __syncthreads();
  const int n_sel = (int)L.n_sel < kSortCap ? (int)L.n_sel : kSortCap;
  const int n_ties = (int)L.n_ties < kTieCap ? (int)L.n_ties : kTieCap;
  if ((uint32_t)n_ties > need_t) {  // keep the need_t smallest indices among the ties
    const int p2 = pow2_at_least(n_ties);
    for (int i = n_ties + t; i < p2; i += kSelThreads) L.ties[i] = 0xffffffffu;
    __syncthreads();
    bitonic_u32(L.ties, p2);
  }
  for (int i = t; i < (int)need_t; i += kSelThreads) {
    if (n_sel + i < kSortCap) { L.skey[n_sel + i] = T; L.sidx[n_sel + i] = L.ties[i]; }
  }
  __syncthreads();
  const int n_all = n_sel + (int)need_t < kSortCap ? n_sel + (int)need_t : kSortCap;
  order_store(L.skey, L.sidx, n_all, (uint64_t*)L.ties, out);
  for (int i = n_all + t; i < topk; i += kSelThreads) out[i] = -1;
}

}  // namespace

size_t topk_ws_bytes(int64_t R) {
  size_t b = align_up((size_t)R * kHistBins * 4, 256);
  b += align_up((size_t)R * 32, 256);
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
  p += align_up((size_t)R * 32, 256);
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
  static_assert(sizeof(RowInfo) <= 32, "row info slot");
  // at least kCollectWgs work-groups where the rows allow it
  constexpr int64_t kCollectWgs = 512;
  int ch = kChunk;
  while (ch > kChunk / 4 && R * ((ld + ch - 1) / ch) < kCollectWgs) ch >>= 1;
  const int64_t gx = (ld + ch - 1) / ch;
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    const dim3 grid((unsigned)gx, (unsigned)nr);
    auto args = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(kSelThreads), 0, s, scores + r0 * ld, n_valid + r0, ld,
                         topk, w.hist + r0 * kHistBins, (RowInfo*)w.ctr + r0,
                         w.cand + r0 * (int64_t)kCandCap * 2, w.hi + r0 * (int64_t)kTopkMax * 2);
    };
    if (ch == kChunk) args(topk_collect_kernel<kChunk>);
    else if (ch == kChunk / 2) args(topk_collect_kernel<kChunk / 2>);
    else args(topk_collect_kernel<kChunk / 4>);
  }
  for (int64_t r0 = 0; r0 < R; r0 += 65535) {
    int64_t nr = R - r0 < 65535 ? R - r0 : 65535;
    hipLaunchKernelGGL(topk_final_kernel, dim3(2u, (unsigned)nr), dim3(kSelThreads), 0, s,
                       scores + r0 * ld, n_valid + r0, ld, topk, out_idx + r0 * topk,
                       (const RowInfo*)w.ctr + r0, w.cand + r0 * (int64_t)kCandCap * 2,
                       w.hi + r0 * (int64_t)kTopkMax * 2);
  }
  return hipGetLastError();
}

}  // namespace csa
