// The expert FFN for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the same kernels as moeq_expert_ffn, with the working
// memory taken from a fixed device array instead of a caller workspace.
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy until the process ends.  In host code
// its name is only a host-side stand-in, so its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// only that address is handed to the kernels.
#include <mutex>
#include "common.hpp"

namespace moeq {

constexpr size_t kScratchBytes = (size_t)64 << 20;     // 64 MiB per device
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void *g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on first use).
static moeq_status scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOEQ_ERR_HIP, "expert_ffn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOEQ_ERR_UNSUPPORTED, "expert_ffn_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOEQ_ERR_HIP, "expert_ffn_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOEQ_OK;
}

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_ffn_noalloc_max_bytes(size_t *bytes) {
  if (!bytes) return fail(MOEQ_ERR_INVALID, "ffn_noalloc_max_bytes: null argument");
  *bytes = kScratchBytes;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_expert_ffn_noalloc(const moeq_layer *L, const uint16_t *x, int32_t T, int32_t k,
                                             const moeq_routing *r, int32_t n_comp, void *y, int32_t y_dtype,
                                             const moeq_ffn_options *opts, hipStream_t stream) {
  size_t need = 0;
  moeq_status st = moeq_ffn_workspace_size(L, T, k, opts, &need);
  if (st != MOEQ_OK) return st;
  if (need > kScratchBytes)
    return fail(MOEQ_ERR_WORKSPACE,
                "expert_ffn_noalloc: this call needs %zu bytes of working memory, more than the %zu of the "
                "fixed device array (use moeq_expert_ffn with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  if (T > 0) {
    st = scratch_ptr(&ws);
    if (st != MOEQ_OK) return st;
  }
  return moeq_expert_ffn(L, x, T, k, r, n_comp, y, y_dtype, ws, kScratchBytes, opts, stream);
}
