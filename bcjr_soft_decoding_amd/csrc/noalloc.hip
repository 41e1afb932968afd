// Forward without a workspace argument, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The forward's message history (the only scratch it uses) lives in a fixed array of this
// library's code object, `scratch`, which the runtime places in device memory on every device
// the library runs on and keeps until the process ends. Its host-side name is not a device
// address: the first call on a device looks the address up with hipGetSymbolAddress (with that
// device current) and keeps it per device; kernels only ever receive that address, as the
// workspace of the ordinary forward, whose kernels and validation this entry point shares.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bcjr.h"

namespace {

constexpr size_t kScratchBytes = BCJR_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size is a multiple of its alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, under g_mu

// The current device's scratch address, looked up on the first call on that device.
bcjr_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BCJR_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return BCJR_E_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return BCJR_OK;
}

}  // namespace

extern "C" bcjr_status bcjr_forward_noalloc(const bcjr_trellis* tr, const float* w, int64_t B,
                                            int64_t L, float T, float* w_hat, float* log_z,
                                            void* saved, bcjr_stream_t stream) {
  // Shapes whose smallest (checkpointed) history exceeds the array are refused before any
  // device call; the size query returns 0 for invalid shapes, which the forward then reports.
  if (bcjr_workspace_bytes(tr, B, L, 3) > kScratchBytes) return BCJR_E_WORKSPACE;
  void* ws = nullptr;
  const bcjr_status st = scratch_on_current_device(&ws);
  if (st != BCJR_OK) return st;
  // the full history where it fits the array, else the checkpointed one (bitwise the same)
  return bcjr_forward(tr, w, B, L, T, w_hat, log_z, saved, ws, kScratchBytes, stream);
}
