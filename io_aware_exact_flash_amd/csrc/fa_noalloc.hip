// flash_attn_bwd_noalloc: the backward pass with its workspace in memory the
// library holds, for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that must not call hipMalloc, harnesses
// that forbid it).
//
// The backward's workspace (two float32 values per query row: D_i =
// rowsum(dO o O) and the base-2 log-sum-exp) lives in `scratch`, a
// file-scope device array of kScratchBytes.  Each GPU holds its own copy at
// its own address; that address is looked up once per device with
// hipGetSymbolAddress and kept, and only that address ever reaches a kernel
// (in host code the array's name is not a device address).  Every call on a
// GPU shares that GPU's array: calls that overlap on one GPU (on different
// streams) race and give undefined results.  Nothing in the array needs to
// start at zero: the D pre-pass writes every row the other passes read (a
// ragged last tile's 16-byte loads may touch up to 12 spare bytes past an
// array; those values never reach a result).
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_api_internal.hpp"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each GPU

// Workspace supplier for the backward: the calling GPU's copy of `scratch`.
// Runs after every argument check.  The stream (if not the null stream)
// must belong to the current device, on which the address is looked up.
// Allocates nothing.
fa_status scratch_workspace(const char* fn, size_t need, hipStream_t stream, void** ws, size_t* bytes) {
  if (need > kScratchBytes)
    return fa::fail_status(FA_ERR_UNSUPPORTED,
                           "%s: the problem needs %zu bytes of workspace, more than the %zu this call holds "
                           "per GPU (use flash_attn_bwd with a caller-provided workspace)",
                           fn, need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa::fail_status(FA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (stream) {
    // the kernels run on the stream's device and the array's address is
    // looked up on the current one: the two must agree
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fa::fail_status(FA_ERR_HIP, "%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
    if (sdev != dev)
      return fa::fail_status(FA_ERR_INVALID_ARGUMENT, "%s: stream belongs to device %d, current device is %d", fn,
                             sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fa::fail_status(FA_ERR_UNSUPPORTED, "%s: device index %d outside 0..%d", fn, dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fa::fail_status(FA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                             hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  *bytes = kScratchBytes;
  return FA_OK;
}

}  // namespace

FA_EXPORT fa_status flash_attn_bwd_noalloc(int B, int H, int N, int d, fa_dtype dtype, const void* q, const void* k,
                                           const void* v, const void* o, const void* dout, const float* lse,
                                           float scale, int causal, void* dq, void* dk, void* dv,
                                           hipStream_t stream) {
  return fa::bwd_dense_with("flash_attn_bwd_noalloc", B, H, N, d, dtype, q, k, v, o, dout, lse, scale, causal, dq, dk, dv,
                            scratch_workspace, stream);
}
