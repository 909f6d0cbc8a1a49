// moe_fused_dev.h -- device helpers of the single-token kernels (the
// one-layer launch k_layer1 and the multi-layer launch k_stack): launch
// geometry, coherent and buffer loads, LDS flags between the waves of a
// workgroup, the fp8 pair convert of the down products and the down-row
// partial sums.  Included by moe_fused.hip and moe_stack.hip (each gets its
// own copy in an unnamed namespace).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kG = 256;          // workgroups
constexpr int kGuWaves = 4;      // gate/up waves 0..3
constexpr int kDownWaves = 4;    // down waves 4..7 (wave 4 runs the exchange)
constexpr int kNT = 64 * (kGuWaves + kDownWaves);
constexpr long kSpinMax = 1L << 18;
constexpr float kRmsEps = 1e-6f;  // epsilon of the pre-MoE RMS norm

// LDS layouts of the activations h and the packed x pairs, swizzled per
// 16-byte chunk (1) or plain (0).  A reader lane takes one run of 16-byte
// chunks (h: 32 values of one down lane; x pairs: one gate/up segment) and the
// runs of neighbouring lanes are 64 or 128 bytes apart, so the lanes of one
// ds_read_b128 would all hit the same banks; storing chunk c of run n at
// chunk position c ^ key(n) spreads them over all banks.  Only addresses
// change: every value is read into the same register as before.
#ifndef MOE_LDS_SWIZZLE
#define MOE_LDS_SWIZZLE 1
#endif
// Float position of element i of one slot's h (runs of 32 floats = 8 chunks).
__device__ __forceinline__ int hb_pos(int i) {
  return MOE_LDS_SWIZZLE ? (i ^ (((i >> 5) & 7) << 2)) : i;
}
// XOR applied to the float offsets within down lane `seg`'s run of h.
__device__ __forceinline__ int hb_key(int seg) { return MOE_LDS_SWIZZLE ? (seg & 7) << 2 : 0; }
// Word position of pair j of x segment sg (PAIRS words per segment).
template <int PAIRS>
__device__ __forceinline__ int xp_key(int sg) {
  static_assert(PAIRS == 16 || PAIRS == 32, "4 or 8 chunks per segment");
  if (!MOE_LDS_SWIZZLE) return 0;
  return (PAIRS == 32 ? (sg & 7) : ((sg >> 1) & 3)) << 2;
}

typedef __attribute__((address_space(3))) volatile uint32_t lds_u32;

__device__ __forceinline__ lds_u32 *lds(uint32_t *p) { return (lds_u32 *)(p); }
typedef __attribute__((address_space(3))) volatile float lds_f32;
__device__ __forceinline__ lds_f32 *lds(float *p) { return (lds_f32 *)(p); }

// Ordering of LDS accesses between waves of the workgroup only: these wait
// for outstanding LDS operations, never for global loads.
__device__ __forceinline__ void lds_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}
__device__ __forceinline__ void lds_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Bounded wait until an LDS word written by another wave reaches `want`.
__device__ __forceinline__ void wait_lds(uint32_t *p, uint32_t want) {
  long spins = 0;
  while (*lds(p) < want) {
    if (++spins > (kSpinMax << 4)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_acquire();
}

__device__ __forceinline__ uint32_t ld_rlx(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte coherent load (buffer_load_dwordx4 with the sc1 policy, the same
// policy as an agent-scope relaxed atomic load), coalesced across the wave.
__device__ __forceinline__ uint4 ld_coh16(const void *base, uint32_t byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16 /* sc1 */);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Polling with NP requests in flight.  A coherent poll takes about a
// microsecond to come back; one that finds the data incomplete would cost a
// whole round trip more.  Here the first M polls are issued GAP sleep units
// (64 clocks each) apart with NP of them in flight: they are checked in
// issue order and each incomplete one is followed at once by the next, so
// completion is seen about one round trip after it happens, plus up to one
// gap.  (The M polls are straight-line code: the compiler keeps no load in
// flight across a loop back-edge, where it would copy the registers and wait
// for the load first.)  After them, one poll at a time until the budget runs
// out.
//   issue(u): loads one poll's words into u (NW 16-byte words per lane)
//   ok(u):    whether they are complete (the same on every lane)
//   take(u):  consumes them
//   first():  runs once, right after the first poll is issued (e.g. to let
//             other waves queue their loads behind it)
// Returns false when the spin budget runs out (take() then gets the last,
// incomplete, words).  Polls still in flight at the return are left to
// complete; the compiler waits for them before it reuses their registers.
template <int NW>
__device__ __forceinline__ void launder(uint4 (&u)[NW]) {
  // an empty volatile asm that reads and writes the words (each 16-byte word
  // as one 128-bit register operand): the wait for their load lands here,
  // and nothing computed from them moves above it
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    u32x4 v = {u[i].x, u[i].y, u[i].z, u[i].w};
    __asm__ volatile("" : "+v"(v));
    u[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
template <int NP, int M, int GAP, int NW, typename Issue, typename Ok, typename Take,
          typename First>
__device__ __forceinline__ bool poll_pipe(Issue &&issue, Ok &&ok, Take &&take, long &spins,
                                          First &&first) {
  static_assert(NP >= 1 && M >= NP, "M polls, NP of them in flight");
  uint4 u[NP][NW];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (j) __builtin_amdgcn_s_sleep(GAP);
    // (the barrier keeps the compiler from merging a poll with an earlier
    // one of the same words)
    __asm__ volatile("" ::: "memory");
    issue(u[j]);
    if (j == 0) first();
  }
  // (a complete poll returns at once: a path that went on would meet the
  // path that issued a poll again, and the compiler would copy the words in
  // flight there, waiting for them)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = m % NP;
    launder(u[j]);
    if (ok(u[j])) {
      take(u[j]);
      return true;
    }
    if (m + NP < M) {
      __asm__ volatile("" ::: "memory");
      issue(u[j]);
    }
  }
  spins += M;
  uint4 w[NW];
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    __asm__ volatile("" ::: "memory");
    issue(w);
    launder(w);
    if (ok(w)) {
      take(w);
      return true;
    }
    if (++spins > kSpinMax) {
      take(w);
      return false;
    }
  }
}

template <int NP, int M, int GAP, int NW, typename Issue, typename Ok, typename Take>
__device__ __forceinline__ bool poll_pipe(Issue &&issue, Ok &&ok, Take &&take, long &spins) {
  return poll_pipe<NP, M, GAP, NW>(issue, ok, take, spins, [] {});
}

// Top-K over the wave's logits.  Entry j of lane `lane` holds logit
// 128 (j / 2) + 2 lane + (j & 1), value v[j] (NaN, also for padding, ranks
// below every number).  Order: the largest value first, equal values by
// lower index (NaNs among themselves too).  Each round takes the wave maximum
// M of (order key + 1) over the entries not taken yet (a taken entry's key
// is 0), then the wave minimum of the position (j / 2, lane, j & 1) -- the
// index order -- over the entries holding M, and marks that one taken.
// Branch-free: it runs on one wave between the logits poll and the routed
// loads, where every instruction is on the critical path.
template <int K, int NV>
__device__ __forceinline__ void topk_select(const float (&v)[NV], int lane, float (&sel_v)[K],
                                            int (&sel_i)[K]) {
  uint32_t key[NV], pos[NV];  // pos: (j / 2) << 8 | lane << 1 | (j & 1)
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    key[j] = f32_order_key(v[j]) + 1u;  // at most 0xFF800001
    pos[j] = ((uint32_t)(j >> 1) << 8) | ((uint32_t)lane << 1) | (j & 1);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) m = max(m, key[j]);
    const uint32_t M = wave_max_u32(m);  // >= 1: fewer than K entries are taken
    uint32_t c = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < NV; ++j) c = min(c, key[j] == M ? pos[j] : 0xFFFFFFFFu);
    const uint32_t P = wave_min_u32(c);
#pragma unroll
    for (int j = 0; j < NV; ++j) key[j] = pos[j] == P ? 0u : key[j];
    sel_i[k] = (int)((P >> 8) * 128u + (P & 255u));
    const uint32_t ok = M - 1u;
    sel_v[k] = __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
  }
}

// Routing weights of the selection, lane k (< K) computing slot k's:
// w_k = p_k / (p_0 + .. + p_{K-1}), p_k = exp(v_k - v_0), the sum in slot
// order.  id and w are those of slot `lane` on lanes < K.
template <int K>
__device__ __forceinline__ void topk_weights(const float (&sel_v)[K], const int (&sel_i)[K],
                                             int lane, int &id, float &w) {
  float sv = sel_v[0];
  id = sel_i[0];
#pragma unroll
  for (int k = 1; k < K; ++k) {
    sv = lane == k ? sel_v[k] : sv;
    id = lane == k ? sel_i[k] : id;
  }
  const float p = expf(sv - sel_v[0]);
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k)
    den += __uint_as_float((uint32_t)__builtin_amdgcn_readlane(__float_as_uint(p), k));
  w = p / den;
}

// 8-byte coherent load, the same policy.
__device__ __forceinline__ uint2 ld_coh8(const void *base, uint32_t byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 16 /* sc1 */);
  return make_uint2(v[0], v[1]);
}

// Weight loads through a buffer resource of the blob: the per-lane byte
// offsets are the same 32-bit values for every expert, only the (scalar)
// resource changes, which keeps 64-bit address arithmetic out of the vector
// registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t blob_rsrc(const uint8_t *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, 0x7fffffff, 0x00020000);
}
// POL: the cache-policy bits of the load (0: default; kPolStream: the
// non-temporal hint for bytes that are read once)
constexpr int kPolStream = 2;
template <int POL = 0>
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int POL = 0>
__device__ __forceinline__ uint2 bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POL);
  return make_uint2(v[0], v[1]);
}
template <int POL = 0>
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL);
}

template <int BITS, int H, int I, int K>
struct Geo {
  static constexpr int COLS = 128 / BITS;           // columns per 16-byte segment
  static constexpr int PAIRS = COLS / 2;            // packed x pairs per segment
  static constexpr int SEG_X = H * BITS / 128;      // segments per gate/up row
  static constexpr int LSEG = SEG_X / 64;           // segments per lane per gate/up row
  static constexpr int XLD = COLS * 2 / 16;         // 16-byte x loads per segment
  static constexpr int RCH = H / 8;                 // 16-byte chunks per router row
  static constexpr int RXC = RCH / kNT;             // router x chunks per thread
  static constexpr int GU_ROWS = I / kG;            // gate/up rows per workgroup and slot
  static constexpr int DCOLS = 32;                  // down codes per lane (one load)
  static constexpr int DWORDS = DCOLS * BITS / 32;  // their code words (4 or 2)
  static constexpr int LPR = I / DCOLS;             // lanes per down row
  static constexpr int RPL = 64 / LPR;              // down rows per wave-wide load
  static constexpr int NSEGD = 1;
  static constexpr int D_ROWS = H / kG;             // down rows per workgroup
  static constexpr int D_ROWS_W = D_ROWS / kDownWaves;  // per down wave
  static constexpr int DLD = D_ROWS_W / RPL;        // down loads per lane per slot
  static_assert(LSEG >= 1 && SEG_X % 64 == 0, "gate/up row must span a wave");
  static_assert(GU_ROWS == kGuWaves, "one gate/up row per gate/up wave and slot");
  static_assert(LPR <= 64 && 64 % LPR == 0, "a down row within one wave");
  static_assert(DLD >= 1 && D_ROWS_W % RPL == 0, "down rows must tile the waves");
  static_assert(RXC >= 1 && RCH % kNT == 0, "router row must span the workgroup");
  static_assert(SEG_X <= 64 * kGuWaves, "one x segment per gate/up thread");
  // the down rows of each routed slot are split over OWN_WG workgroups
  static constexpr int OWN_WG = kG / K;             // workgroups per routed slot
  static constexpr int O_ROWS = H / OWN_WG;         // routed down rows per workgroup
  static constexpr int O_ROWS_W = O_ROWS / kDownWaves;  // per down wave
  static constexpr int RDLD = O_ROWS_W / RPL;       // routed down loads per lane
  static_assert(kG % K == 0 && H % OWN_WG == 0, "routed rows must tile the workgroups");
  static_assert(RDLD >= 1 && O_ROWS_W % RPL == 0 && O_ROWS_W <= 64, "routed rows per wave");
  static_assert(K * D_ROWS == 64, "one routed sum per lane of the exchange wave");
};


// Value of code 1 read as an fp8 bit pattern.  A masked code byte (0..15)
// is an fp8 subnormal or the smallest normals, so its fp8 value is exactly
// the code times this power of two (2^-9 for e4m3, 2^-10 for its FNUZ form).
__device__ __forceinline__ float fp8_code_unit() {
  return __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
}

// The codes of one 32-bit word of a down row as fp32 values u q_c, in column
// order (8 at 4 bits, 16 at 2 bits), u = fp8_code_unit().  m is the per-byte
// code mask (0x0F0F0F0F or 0x03030303) in a register the compiler cannot see
// through.  Each masked word converts two codes per instruction
// (v_cvt_pk_f32_fp8 on its low and high half): at 4 bits the masked word
// holds codes (0, 2, 4, 6) and the word shifted by 4 codes (1, 3, 5, 7); at
// 2 bits the word shifted by 2k holds codes (k, 4 + k, 8 + k, 12 + k).
// This is the unpack of the single-token down products (word_dot_f32); the
// dequantisation hook (moe_dequantize_as) calls it too.
template <int BITS>
__device__ __forceinline__ void fp8_word_codes(uint32_t u, uint32_t m, float (&q)[32 / BITS]) {
  if (BITS == 4) {
    const uint32_t lo = u & m, hi = (u >> 4) & m;
    const auto l0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const auto l1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const auto h0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const auto h1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    q[0] = l0[0];
    q[1] = h0[0];
    q[2] = l0[1];
    q[3] = h0[1];
    q[4] = l1[0];
    q[5] = h1[0];
    q[6] = l1[1];
    q[7] = h1[1];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t mk = (u >> (2 * k)) & m;
      const auto c0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)mk, false);
      const auto c1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)mk, true);
      q[k] = c0[0];
      q[4 + k] = c0[1];
      q[8 + k] = c1[0];
      q[12 + k] = c1[1];
    }
  }
}

// u sum_c q_c h_c over the codes of one 32-bit word of a down row, fp32; hv
// holds the word's activations.  The products are summed in the order the
// conversions produce them (column order at 4 bits; k-major at 2 bits); u is
// a power of two, so the sum is exactly u times the one formed from integer
// codes.
template <int BITS>
__device__ __forceinline__ float word_dot_f32(uint32_t u, const float *hv, float acc, uint32_t m) {
  float q[32 / BITS];
  fp8_word_codes<BITS>(u, m, q);
  if (BITS == 4) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc = fmaf(q[c], hv[c], acc);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(q[k], hv[k], acc);
      acc = fmaf(q[4 + k], hv[4 + k], acc);
      acc = fmaf(q[8 + k], hv[8 + k], acc);
      acc = fmaf(q[12 + k], hv[12 + k], acc);
    }
  }
  return acc;
}

// Lane partial sums of N down rows, one code load per row and lane, against
// the activations of the lane's DCOLS columns (hb, in LDS, offsets XOR key):
// acc += wk (s sum_c q_c h_c + z sum_c h_c) with the row's group scale s and
// bias z.  One code word's activations are read from LDS at a time.
template <int BITS, int N, int DWORDS, int DCOLS>
__device__ __forceinline__ void down_rows(const uint4 (&dq)[N], const uint32_t (&dsb)[N],
                                          const float *hb, int key, float wk, float (&acc)[N]) {
  constexpr int CPW = 32 / BITS;  // codes per word
  uint32_t m = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  asm volatile("" : "+s"(m));
  static_assert(CPW * DWORDS == DCOLS, "the lane's codes fill its words");
  float q[N];
#pragma unroll
  for (int ld = 0; ld < N; ++ld) q[ld] = 0.f;
  float Hs = 0.f;
#pragma unroll
  for (int wd = 0; wd < DWORDS; ++wd) {
    float hv[CPW];
#pragma unroll
    for (int t = 0; t < CPW / 4; ++t) {
      const float4 v = *reinterpret_cast<const float4 *>(hb + ((CPW * wd + 4 * t) ^ key));
      hv[4 * t] = v.x;
      hv[4 * t + 1] = v.y;
      hv[4 * t + 2] = v.z;
      hv[4 * t + 3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) Hs += hv[c];
#pragma unroll
    for (int ld = 0; ld < N; ++ld) {
      const uint4 c4 = dq[ld];
      const uint32_t u = wd == 0 ? c4.x : wd == 1 ? c4.y : wd == 2 ? c4.z : c4.w;
      q[ld] = word_dot_f32<BITS>(u, hv, q[ld], m);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // q holds u times the integer-code sums; 1/u is exact
  const float iu = 1.f / fp8_code_unit();
#pragma unroll
  for (int ld = 0; ld < N; ++ld) {
    const uint32_t sb = dsb[ld];
    acc[ld] += wk * (bf16f(sb & 0xFFFFu) * iu * q[ld] + bf16f(sb >> 16) * Hs);
  }
}

// Sums of the two 32-lane halves of a wave, uniform across the wave.
__device__ __forceinline__ void half_sums32(float v, float &lo, float &hi) {
  v = row16_sum(v);
  lo = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0)) +
       __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  hi = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32)) +
       __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
}

// Sum over aligned groups of LPR lanes (16, 32 or 64) without LDS traffic.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v, int lane) {
  static_assert(LPR == 16 || LPR == 32 || LPR == 64, "group of 16, 32 or 64 lanes");
  if (LPR == 16) return row16_sum(v);
  if (LPR == 32) return half_sum32(v, lane);
  return wave_sum64(v);
}

}  // namespace
}  // namespace moe
