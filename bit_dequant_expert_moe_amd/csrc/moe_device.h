// moe_device.h -- device helpers shared by the gfx950 kernels: bf16/fp16
// conversions, the packed-pair nibble unpack, dot products and reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {
namespace dev {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  h2_t v;
  v.x = (_Float16)lo;
  v.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float h2_sum(uint32_t p) {
  h2_t v = __builtin_bit_cast(h2_t, p);
  return (float)v.x + (float)v.y;
}

// (w & m) | c in one VALU op (the compiler would otherwise emit AND and OR
// with two literal operands).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c,
                                false);
}

__device__ __forceinline__ float dot2b(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a),
                                         __builtin_bit_cast(b2_t, b), c, false);
}

// ---- cross-lane operations on DPP row permutes (no LDS traffic) -------------
// dpp_ctrl codes (gfx9): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141 (lane i <- 7-i in each 8), row_mirror = 0x140
// (lane i <- 15-i in each row of 16).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(dpp_u<CTRL>(__float_as_uint(v)));
}

// Sum of each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// Sum over the 64 lanes of the wave (wave-uniform result).
__device__ __forceinline__ float wave_sum64(float v) {
  v = row16_sum(v);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0)) +
         __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16)) +
         __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32)) +
         __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
}

// Sum over each half of the wave (lanes 0-31, 32-63); result valid in all lanes.
__device__ __forceinline__ float half_sum32(float v, int lane) {
  v = row16_sum(v);
  const float lo = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0)) +
                   __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float hi = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32)) +
                   __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return lane < 32 ? lo : hi;
}

// Maximum of a 64-bit key over the wave (wave-uniform result).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  auto step = [&](auto ctrl_tag) {
    constexpr int C = decltype(ctrl_tag)::value;
    const uint32_t lo = dpp_u<C>((uint32_t)k), hi = dpp_u<C>((uint32_t)(k >> 32));
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    k = o > k ? o : k;
  };
  step(std::integral_constant<int, 0xB1>{});
  step(std::integral_constant<int, 0x4E>{});
  step(std::integral_constant<int, 0x141>{});
  step(std::integral_constant<int, 0x140>{});
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t o = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(k >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((uint32_t)k, 16 * r);
    m = o > m ? o : m;
  }
  return m;
}

// Maximum of a 32-bit value over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = max(k, dpp_u<0xB1>(k));
  k = max(k, dpp_u<0x4E>(k));
  k = max(k, dpp_u<0x141>(k));
  k = max(k, dpp_u<0x140>(k));
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane(k, 0);
  m = max(m, (uint32_t)__builtin_amdgcn_readlane(k, 16));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane(k, 32));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane(k, 48));
  return m;
}

// Minimum of a 32-bit value over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t k) {
  k = min(k, dpp_u<0xB1>(k));
  k = min(k, dpp_u<0x4E>(k));
  k = min(k, dpp_u<0x141>(k));
  k = min(k, dpp_u<0x140>(k));
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane(k, 0);
  m = min(m, (uint32_t)__builtin_amdgcn_readlane(k, 16));
  m = min(m, (uint32_t)__builtin_amdgcn_readlane(k, 32));
  m = min(m, (uint32_t)__builtin_amdgcn_readlane(k, 48));
  return m;
}

// Order-preserving map of an fp32 value to uint32 (NaN -> 0, i.e. below all).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  if (f != f) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum over aligned groups of `width` lanes (power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

constexpr uint32_t kMagicH = 0x64006400u;  // fp16 pair (1024, 1024)
constexpr uint32_t kMagicB = 0x43004300u;  // bf16 pair (128, 128)

// ---------------------------------------------------------------------------
// x staging for the gate/up GEMV.  For each 16-byte code segment of a row
// (32 codes at 4 bits, 64 at 2 bits) the LDS holds the packed fp16 x pairs in
// the order the unpack produces them, plus two floats:
//   C = 1024 * (sum of the fp16 values of the pairs)   (removes the magic)
//   X = sum of x over the segment's columns            (bias term)
// ---------------------------------------------------------------------------
template <int BITS>
struct XSeg {
  static constexpr int kCols = 128 / BITS;      // columns per segment
  static constexpr int kPairs = kCols / 2;      // packed pairs per segment
};

template <int BITS>
__device__ void stage_x(const uint16_t *__restrict__ x, int H, uint32_t *xp, float2 *cx) {
  constexpr int kCols = XSeg<BITS>::kCols, kPairs = XSeg<BITS>::kPairs;
  const int nseg = H / kCols;
  for (int sg = threadIdx.x; sg < nseg; sg += blockDim.x) {
    const uint16_t *xs = x + sg * kCols;
    float C = 0.f, X = 0.f;
    for (int wd = 0; wd < 4; ++wd) {
      if (BITS == 4) {
        // word wd holds codes 8wd .. 8wd+7; pairs (0,4) (1,5)/16 (2,6) (3,7)/16
        float v[8];
        for (int j = 0; j < 8; ++j) v[j] = bf16f(xs[8 * wd + j]);
        for (int j = 0; j < 8; ++j) X += v[j];
        const float sc[4] = {1.f, 0.0625f, 1.f, 0.0625f};
        for (int p = 0; p < 4; ++p) {
          uint32_t pr = pack_h2(v[p] * sc[p], v[p + 4] * sc[p]);
          xp[sg * kPairs + 4 * wd + p] = pr;
          C += h2_sum(pr);
        }
      } else {
        // word wd holds codes 16wd .. 16wd+15; pair k = (k, k+8) scaled by
        // 4^-k (k < 5) or 4^-(k-5) (k >= 5, taken from the word shifted by 10)
        float v[16];
        for (int j = 0; j < 16; ++j) v[j] = bf16f(xs[16 * wd + j]);
        for (int j = 0; j < 16; ++j) X += v[j];
        for (int k = 0; k < 8; ++k) {
          const int e = k < 5 ? k : k - 5;
          const float sc = 1.f / (float)(1 << (2 * e));
          uint32_t pr = pack_h2(v[k] * sc, v[k + 8] * sc);
          xp[sg * kPairs + 8 * wd + k] = pr;
          C += h2_sum(pr);
        }
      }
    }
    cx[sg] = make_float2(1024.f * C, X);
  }
}

// Packed fp16 pair p of one 32-bit code word: (1024 + m q_a, 1024 + m q_b)
// with one v_and_or_b32 against the magic 0x6400 (1024.0).  The pair holds
//   4 bits: codes (p, p + 4) of the word's 8, with m = 16^(p & 1);
//   2 bits: codes (p, p + 8) of the word's 16, with m = 4^p (p < 5) or
//           4^(p - 5) (p >= 5, fields taken from the word shifted by 10).
// 1024 + m q is exact in fp16 (m q <= 256 < 1024 = its unit step times 2^10).
// This is the unpack of the single-token gate/up products (seg_dot_x); the
// dequantisation hook (moe_dequantize_as) calls it too.
// (us is the word shifted right by 8 at 4 bits, by 10 at 2 bits; the caller
// forms it once per word.)
template <int BITS>
__device__ __forceinline__ uint32_t h2_code_pair(uint32_t u, uint32_t us, int p) {
  const uint32_t M = kMagicH;
  if (BITS == 4) {
    return and_or(p < 2 ? u : us, (p & 1) ? 0x00F000F0u : 0x000F000Fu, M);
  } else {
    const int f = p < 5 ? p : p - 5;
    return and_or(p < 5 ? u : us, 0x00030003u << (2 * f), M);
  }
}
template <int BITS>
__device__ __forceinline__ uint32_t h2_shifted(uint32_t u) {
  return BITS == 4 ? u >> 8 : u >> 10;
}

// sum_c (magic_c + q_c) * xtilde_c over one 16-byte segment.
template <int BITS>
__device__ __forceinline__ float seg_dot_x(uint4 c, const uint32_t *xp) {
  constexpr int NP = 16 / BITS;  // pairs per word (4 or 8)
  float acc = 0.f;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t us = h2_shifted<BITS>(w[wd]);
      acc = dot2h(h2_code_pair<BITS>(w[wd], us, p), xp[NP * wd + p], acc);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Dequantisation hooks (moe_dequantize, moe_dequantize_as): one matrix of a
// blob as fp32, one thread per 32-bit code word, each code decoded by the
// unpack of one kernel path.
// ---------------------------------------------------------------------------
struct DequantArgs {
  const uint32_t *q, *sb;  // the matrix's code words [rows][cols / cpw] and (s, z) words
  float *out;              // fp32 [rows][cols]
  int rows, cols, bits;
};

// Writes s q_j + z for the CPW codes of word (r, c0 / CPW), q in column
// order as exact integers in fp32: s q is exact in fp32 (8 significant bits
// times at most 4), so the FMA rounds the exact value s q + z once.
template <int CPW>
__device__ __forceinline__ void store_dequant_word(const DequantArgs &a, size_t r, int c0,
                                                   const float (&q)[CPW]) {
  const uint32_t sz = a.sb[r * (a.cols / 64) + c0 / 64];
  const float s = bf16f(sz & 0xFFFFu), z = bf16f(sz >> 16);
  float *o = a.out + r * a.cols + c0;
#pragma unroll
  for (int j = 0; j < CPW; ++j) o[j] = fmaf(s, q[j], z);
}

}  // namespace dev
}  // namespace moe
