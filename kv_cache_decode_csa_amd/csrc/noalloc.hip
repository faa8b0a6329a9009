// csa_index_topk_noalloc: the index + top-k call with its scratch memory in a
// fixed device array owned by the library, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid allocation).  The arithmetic is csa_index_topk's: this file only
// supplies the scratch.
#include <mutex>

#include "csa_internal.h"

namespace {

// Every device the library runs on holds its own copy of this array until the
// process ends.  32 MiB covers 8 sequences of 262,144 entries (9.2 MB) and, at
// that length, up to 28 query rows (B * Q).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address per device, resolved once with that device
// current.  In host code `scratch` is only a stand-in symbol, never an
// address; kernels receive the resolved pointer.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

extern "C" csa_status csa_index_topk_noalloc(const void* q_idx, int q_fmt, const float* w_idx,
                                             const void* k_idx, int k_fmt, const int32_t* pos,
                                             int ratio, int B, int Q, int Hi, int64_t Nmax,
                                             int topk, int32_t* out_idx, float* out_scores,
                                             csa_stream_t stream) {
  const size_t need = csa_index_topk_workspace_size(B, Q, Nmax, topk);
  if (need > kScratchBytes)
    return csa::set_error(CSA_EWORKSPACE,
                          "csa_index_topk_noalloc: B=%d Q=%d Nmax=%lld needs %zu bytes of "
                          "scratch; the library's fixed scratch holds %zu",
                          B, Q, (long long)Nmax, need, kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return csa::set_error(CSA_ELAUNCH, "csa_index_topk_noalloc: hipGetDevice: %s",
                          hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return csa::set_error(CSA_EUNSUPPORTED, "csa_index_topk_noalloc: device %d >= %d", dev,
                          kMaxDevices);
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return csa::set_error(CSA_ELAUNCH, "csa_index_topk_noalloc: hipGetSymbolAddress: %s",
                              hipGetErrorString(e));
      g_scratch[dev] = p;
    }
    ptr = g_scratch[dev];
  }
  // csa_index_topk validates every argument before it enqueues anything and
  // clears the counters it needs with a kernel, so stale contents from the
  // previous call on this device do not matter.
  return csa_index_topk(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk,
                        out_idx, out_scores, ptr, kScratchBytes, stream);
}
