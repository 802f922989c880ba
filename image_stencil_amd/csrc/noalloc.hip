// noalloc.hip -- conv_chain_forward_noalloc: the chain entry point with a
// workspace the library owns, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The layer-by-layer chain keeps its intermediate tensors in a workspace. Here
// that workspace is a file-scope device array of kScratchBytes, which the code
// object loader places on every device that loads this library, once, for the
// life of the process. Host code never uses the array's name as an address
// (in host code it names a host-side stand-in): the device address of the
// current device's copy comes from hipGetSymbolAddress, once per device, and
// only that address is passed on.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace {

// Enough for the layer-by-layer chains of a 1280x720 frame: two 32-channel
// fp32 intermediates (2 x 118 MB) or two 64-channel fp16 ones (2 x 118 MB).
constexpr size_t kScratchBytes = IS_NOALLOC_MAX_WORKSPACE;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The current device's copy of the scratch array; the stream must belong to
// that device (the array's address differs per device).
is_status scratch_for(hipStream_t stream, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return is::report_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return IS_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return is::report_hip(e);
    if ((int)sdev != dev) return IS_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return is::report_hip(e);
    if (!p) return IS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return IS_OK;
}

}  // namespace

extern "C" {

is_status conv_chain_forward_noalloc(const conv_chain_desc *d, const void *x, const void *const *w,
                                     const float *const *b, void *y, hipStream_t stream) {
  try {
    size_t need = 0;
    const is_status st = conv_chain_workspace_size(d, &need);   // validates d, host only
    if (st != IS_OK) return st;
    if (need > kScratchBytes) return IS_ERR_WORKSPACE;
    if (!x || !w || !y) return IS_ERR_INVALID_ARG;
    void *ws = nullptr;
    if (need > 0) {
      const is_status s2 = scratch_for(stream, &ws);
      if (s2 != IS_OK) return s2;
    }
    // The intermediates need no clearing: every layer writes all of its output
    // before the next layer reads it.
    return is::chain_forward(d, x, w, b, y, ws, need > 0 ? kScratchBytes : 0, stream);
  } catch (...) {
    return IS_ERR_INVALID_ARG;
  }
}

}  // extern "C"
