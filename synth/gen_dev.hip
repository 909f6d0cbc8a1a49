// gen_dev.hip -- device build of the synthetic expert-blob generator
// (synth_common.h).  Fills n consecutive expert blobs in device memory; the
// bytes equal those of gen_host.c for the same (params, layer, expert).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_common.h"

namespace {

struct GenArgs {
  synth_params p;
  uint64_t off[7];
  uint8_t *dst;
  int64_t stride;  // bytes between consecutive blobs
  uint32_t layer, e0;
  int32_t n;
  uint64_t quads;  // 16-byte chunks per blob (blob words / 4)
};

__global__ void __launch_bounds__(256) k_gen_blobs(GenArgs a) {
  const uint64_t total = a.quads * (uint64_t)a.n;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t e = q / a.quads;
    const uint64_t w = (q - e * a.quads) * 4;
    const uint64_t key = synth_key(a.p.seed, a.layer, a.e0 + (uint32_t)e);
    uint4 v;
    v.x = synth_blob_word(&a.p, key, a.off, w + 0);
    v.y = synth_blob_word(&a.p, key, a.off, w + 1);
    v.z = synth_blob_word(&a.p, key, a.off, w + 2);
    v.w = synth_blob_word(&a.p, key, a.off, w + 3);
    *reinterpret_cast<uint4 *>(a.dst + e * a.stride + w * 4) = v;
  }
}

}  // namespace

// Returns 0 on success, -1 on bad arguments, -2 on a HIP error.
extern "C" int synth_gen_blobs_dev(const synth_params *p, uint32_t layer,
                                   uint32_t e0, int32_t n, void *dst,
                                   int64_t stride, void *stream) {
  if (!p || !dst || n < 0) return -1;
  if (n == 0) return 0;
  GenArgs a;
  a.p = *p;
  const uint64_t words = synth_layout(p->H, p->I, p->bits, a.off);
  if (words % 4 != 0 || (uint64_t)stride < words * 4 || stride % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return -1;
  a.dst = static_cast<uint8_t *>(dst);
  a.stride = stride;
  a.layer = layer;
  a.e0 = e0;
  a.n = n;
  a.quads = words / 4;
  const uint64_t total = a.quads * (uint64_t)n;
  uint64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_gen_blobs, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
