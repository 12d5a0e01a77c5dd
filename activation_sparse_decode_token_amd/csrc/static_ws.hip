// spax_layer_step_static: the layer step for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its scratch -- the arrival counters and sync words every launch
// form uses, and the partial sums of split tiles -- lives in one file-scope
// device array of kStaticScratchBytes, which each GPU the library runs on
// holds until the process ends. The array's device address is taken once
// per device with hipGetSymbolAddress; host code never passes the array's
// name itself to a kernel or a copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "spax.h"
#include "spax_internal.h"

namespace {

using namespace spax;

// Largest workspace a layer may need here (the 70B-shaped FFN layer needs
// 14.1 MiB, the 7B layer 5.5 MiB).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // the array's address on each device

// The array's address on the current device (looked up on first use).
int device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_error(hipGetErrorString(e));
    return SPAX_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_last_error("spax_layer_step_static: device index past the supported range");
    return SPAX_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_last_error(e != hipSuccess ? hipGetErrorString(e)
                                     : "spax_layer_step_static: no scratch address");
      return SPAX_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SPAX_OK;
}

}  // namespace

extern "C" int spax_layer_step_static(const spax_layer* L, const spax_layer_io* io,
                                      hipStream_t stream) {
  if (!L || !io) return SPAX_ENULL;
  const size_t need = spax_layer_workspace_bytes(L);
  if (need == 0) return SPAX_EINVAL;
  if (need > kStaticScratchBytes) {
    set_last_error("spax_layer_step_static: the layer needs a workspace larger than the "
                   "library's 16 MiB static scratch; use spax_layer_step");
    return SPAX_EWORKSPACE;
  }
  void* ws = nullptr;
  const int st = device_scratch(&ws);
  if (st) return st;
  // the counters and sync words start at zero on every call (a fill kernel:
  // no memset node when the caller captures the call in a graph)
  const hipError_t e = launch_clear(ws, workspace_head_bytes(), stream);
  if (e != hipSuccess) {
    set_last_error(hipGetErrorString(e));
    return SPAX_EHIP;
  }
  return spax_layer_step(L, io, ws, kStaticScratchBytes, stream, nullptr);
}
