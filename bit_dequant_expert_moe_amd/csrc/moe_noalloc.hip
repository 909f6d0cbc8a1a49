// moe_noalloc.hip -- the multi-layer residual decode for callers that cannot
// allocate device memory (code under graph capture, serving loops that must
// not call hipMalloc).  Its workspace is a fixed array in the library's own
// device memory: one copy per GPU, set up on the entry point's first call on
// that GPU and held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch is whole 256-byte units");

// The workspace of every call on this GPU.  In host code `scratch` names a
// host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, per device, and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_setup;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device once set up

// Device address of the current device's scratch array.  The first call on a
// device looks the address up and enqueues the clearing of the control words
// on `stream` (the workspace initialisation), so it must not be captured.
moe_status scratch_for(void *stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_setup);
  if (!g_scratch[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess)
      return MOE_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    if (launch_ws_init(p, MOE_NOALLOC_SCRATCH_BYTES, stream) != 0) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_stack_decode_residual_noalloc(const moe_dims *dims,
                                                        const moe_layer *layers,
                                                        int32_t n_layers, float *resid,
                                                        uint16_t *x_out, float *y, int32_t *ids,
                                                        float *w, void *stream) {
  const moe_status st = moe::check_stack_residual(dims, layers, n_layers, resid, x_out, y, ids, w);
  if (st != MOE_OK) return st;
  if (moe::ws_layout(*dims, 1).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  const moe_status sst = moe::scratch_for(stream, &ws);
  if (sst != MOE_OK) return sst;
  return moe_stack_decode_residual(dims, layers, n_layers, resid, x_out, y, ids, w, ws,
                                   MOE_NOALLOC_SCRATCH_BYTES, stream);
}
