// Forward pass for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// hyena_fwd with its workspace taken from a file-scope device array instead of
// a caller buffer. The launch sequence and the kernels are hyena_fwd's own.
#include "../../include/hyena.h"

#include <hip/hip_runtime.h>

#include <mutex>

// One copy per GPU, alive until the process ends. In host code this name is a
// host-side stand-in, not a device address: only the pointer that
// hipGetSymbolAddress returns for the current device may reach a kernel or a
// copy.
__device__ __align__(256) unsigned char scratch[HYENA_NOALLOC_SCRATCH_BYTES];

namespace hy {
// host-side checks of a forward call, defined with hyena_fwd
int fwd_validate(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                 const float* dskip, const void* w_out, int B, int dtype, const void* y, size_t ws_bytes);
}  // namespace hy

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy, resolved once per device.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HYENA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return HYENA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HYENA_OK;
}

}  // namespace

extern "C" int hyena_fwd_noalloc(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                                 const float* dskip, const void* w_out, int B, int dtype, void* y,
                                 hipStream_t stream) {
  // every argument on the host, before any HIP call; a workspace beyond the
  // array is HYENA_ERR_WORKSPACE
  const int chk = hy::fwd_validate(layer, u, w_in, short_w, dskip, w_out, B, dtype, y,
                                   (size_t)HYENA_NOALLOC_SCRATCH_BYTES);
  if (chk != HYENA_OK) return chk;
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st != HYENA_OK) return st;
  // hyena_fwd reads only workspace bytes its own launches wrote earlier in the
  // same call, so the array needs no clearing between calls
  return hyena_fwd(layer, u, w_in, short_w, dskip, w_out, B, dtype, y, ws, (size_t)HYENA_NOALLOC_SCRATCH_BYTES,
                   stream);
}
