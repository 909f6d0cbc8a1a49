// moe_probe.hip -- measurement kernels beside the MoE path (not part of the
// method): a plain streaming read, which measures the HBM read rate one
// launch reaches on this GPU at a given size (the achievable peak that the
// decode kernels are compared with), and a flush, which overwrites the
// 256 MB last-level cache between timed iterations so that a timed launch
// reads its bytes from HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kLoadsInFlight = 8;  // 16-byte loads per thread per round
constexpr size_t kStreamBlocks = 2048;

// Reads `n16` 16-byte words; workgroup b reads the b-th of gridDim.x
// contiguous ranges, kLoadsInFlight coalesced 4 KB blocks per round, and
// writes the XOR of what it read to sink[b] (so that no load can be dropped).
// NT: the loads carry the non-temporal hint.  Measured on this GPU: a
// 2.4 GB stream runs at 6.9 TB/s with it and 5.2 TB/s without, a 40 MB one at
// 2.5 TB/s with it and 4.1 TB/s without; the launcher takes the faster form
// for the size.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint32_t ld_xor(const uint4 *p) {
  if (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  const uint4 v = *p;
  return v.x ^ v.y ^ v.z ^ v.w;
}
constexpr size_t kNtMinBytes = (size_t)256 << 20;  // non-temporal from this size on
template <bool NT>
__global__ void __launch_bounds__(kProbeThreads) k_stream_read(const uint4 *__restrict__ src,
                                                               size_t n16, uint32_t *sink) {
  __shared__ uint32_t s_x[kProbeThreads / 64];
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (kLoadsInFlight - 1) * kProbeThreads < b1; i += kLoadsInFlight * kProbeThreads) {
    uint32_t v[kLoadsInFlight];
#pragma unroll
    for (int k = 0; k < kLoadsInFlight; ++k) v[k] = ld_xor<NT>(src + i + k * kProbeThreads);
#pragma unroll
    for (int k = 0; k < kLoadsInFlight; ++k) acc ^= v[k];
  }
  for (; i < b1; i += kProbeThreads) acc ^= ld_xor<NT>(src + i);
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

// Writes `n16` 16-byte words of `dst` with a value that depends on the index.
__global__ void __launch_bounds__(kProbeThreads) k_flush(uint4 *__restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  for (size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const uint32_t v = (uint32_t)i;
    dst[i] = make_uint4(v, v ^ 0x9E3779B9u, ~v, v + 1u);
  }
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

int stream_read_blocks(size_t bytes) {
  // up to 8 workgroups per compute unit (2048), fewer for small sizes: each
  // reads at least one round of loads
  const size_t per_round = (size_t)kProbeThreads * 16 * kLoadsInFlight;
  size_t b = (bytes + per_round - 1) / per_round;
  if (b > kStreamBlocks) b = kStreamBlocks;
  if (b < 1) b = 1;
  return (int)b;
}

int launch_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (bytes >= kNtMinBytes)
    hipLaunchKernelGGL(k_stream_read<true>, dim3(stream_read_blocks(bytes)), dim3(kProbeThreads),
                       0, S(stream), static_cast<const uint4 *>(src), bytes / 16, sink);
  else
    hipLaunchKernelGGL(k_stream_read<false>, dim3(stream_read_blocks(bytes)), dim3(kProbeThreads),
                       0, S(stream), static_cast<const uint4 *>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

int launch_flush(void *dst, size_t bytes, void *stream) {
  hipLaunchKernelGGL(k_flush, dim3(2048), dim3(kProbeThreads), 0, S(stream),
                     static_cast<uint4 *>(dst), bytes / 16);
  return (int)hipGetLastError();
}

}  // namespace moe
