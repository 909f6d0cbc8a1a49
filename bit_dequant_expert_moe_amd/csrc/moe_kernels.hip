// moe_kernels.hip -- gfx950 kernels of the MoE layer and their launchers.
//
// The method (Flash-MoE pages): "Flash-MoE: Running a 397B Parameter Model on
// a Laptop" (hysenlabs.com), section "How the SSD expert streaming pipeline
// works" -- router, softmax + top-K, the forward pass of the selected
// experts and of the shared expert, combine; "Flash-MoE: Running a 400
// Billion Parameter Model on a MacBook" (mattcullerton.com), section "The
// Architecture" -- 4-bit experts whose dequantisation is folded into the
// FMA inner loop of the matrix-vector product.
//
// Kernels
//   k_router       router logits for T tokens on the matrix cores (bf16 x
//                  bf16 -> fp32, v_mfma_f32_16x16x32_bf16), 16 x 16 tiles.
//   k_router_tiled the same for a large T, 64 x 64 tiles staged in LDS.
//   k_topk         one wave per token: top-K and the renormalised weights.
//   k_gateup       gate and up rows of the selected experts and the shared
//                  expert, SwiGLU epilogue; activations h to the workspace.
//   k_down         down rows of every slot, weighted combine into y.
//   k_dequantize   test hook: one matrix of a blob as fp32.
//
// Inner-loop arithmetic.  A group of 64 weights shares (s, z), so
//   sum_c (s q_c + z) x_c = s * sum_c q_c x_c + z * sum_c x_c,
// and the GEMV needs sum_c q_c x_c only.  Codes are turned into packed
// 16-bit floats with one v_and_or_b32 per pair: OR-ing a 4-bit field into
// the mantissa of 1024.0 (fp16 0x6400) gives 1024 + q (or 1024 + 16 q for a
// field 4 bits up), which v_dot2_f32_f16 multiplies with a pair of x values
// (pre-divided by 16 where the field sits 4 bits up).  The constant 1024 *
// sum x is removed once per 16-byte segment.  The down projection uses the
// same trick in bf16 (128 + q, 0x4300) with h split into bf16 hi + lo so
// that h keeps ~16 significant bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// h staging for the down GEMV: per segment of I (32 or 64 activations) the
// bf16 hi pairs, then the bf16 lo pairs, in the order the unpack produces
// them (4-bit: (j, j+4) for shift 4j; 2-bit: (k, k+8) for shift 2k), plus
//   C = 128 * sum(hi + lo), X = sum h.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ void stage_h(const float *__restrict__ h, int I, uint32_t *hp, float2 *cx) {
  constexpr int kCols = XSeg<BITS>::kCols, kPairs = XSeg<BITS>::kPairs;
  constexpr int kPerWord = 32 / BITS;  // codes per word
  constexpr int kHalf = kPerWord / 2;  // pairs per word
  const int nseg = I / kCols;
  for (int sg = threadIdx.x; sg < nseg; sg += blockDim.x) {
    const float *hs = h + sg * kCols;
    float C = 0.f, X = 0.f;
    for (int wd = 0; wd < 4; ++wd) {
      for (int j = 0; j < kHalf; ++j) {
        const float a = hs[kPerWord * wd + j], b = hs[kPerWord * wd + j + kHalf];
        const uint32_t ah = f2bf(a), bh = f2bf(b);
        const float ar = a - bf16f(ah), br = b - bf16f(bh);
        const uint32_t al = f2bf(ar), bl = f2bf(br);
        hp[sg * 2 * kPairs + kHalf * wd + j] = ah | (bh << 16);
        hp[sg * 2 * kPairs + kPairs + kHalf * wd + j] = al | (bl << 16);
        C += (bf16f(ah) + bf16f(al)) + (bf16f(bh) + bf16f(bl));
        X += a + b;
      }
    }
    cx[sg] = make_float2(128.f * C, X);
  }
}

// bf16 pair j of one code word for the unfused down products:
// (128 + q_a, 128 + q_b) with one v_and_or_b32 against the magic 0x4300
// (128.0); codes (j, j + 4) of 8 at 4 bits, (j, j + 8) of 16 at 2 bits.
// 128 + q is exact in bf16 (q < 16 < 128's unit step times 2^7).  The
// dequantisation hook (moe_dequantize_as) calls it too.
template <int BITS>
__device__ __forceinline__ uint32_t b2_code_pair(uint32_t u, int j) {
  return and_or(u >> (BITS * j), BITS == 4 ? 0x000F000Fu : 0x00030003u, kMagicB);
}

template <int BITS>
__device__ __forceinline__ float seg_dot_h(uint4 c, const uint32_t *hp) {
  constexpr int kPairs = XSeg<BITS>::kPairs;
  constexpr int NP = 16 / BITS;  // pairs per word (4 or 8)
  float acc = 0.f;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const uint32_t v = b2_code_pair<BITS>(w[wd], j);
      acc = dot2b(v, hp[NP * wd + j], acc);
      acc = dot2b(v, hp[kPairs + NP * wd + j], acc);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Routing: logits = W_r x on the matrix cores (bf16 x bf16 products are exact
// in fp32, sums in fp32), then one wave per token selects the top-K.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

struct RouteArgs {
  const uint16_t *router, *x;
  int32_t *ids;
  float *w, *logits_out, *logits;
  int H, E, K, T;
  int S;  // splits of the hidden dimension over blocks (partial logits [S][T][E])
};

// Block = 16 experts x 16 tokens x one of S column ranges; the 4 waves split
// the block's columns and their partial tiles are summed in a fixed order.
// With few tokens the columns are split over S blocks as well, so that the
// router matrix streams through enough workgroups to fill the chip; k_topk
// adds the S partials in order.
__global__ void __launch_bounds__(256) k_router(RouteArgs a) {
  __shared__ f32x4_t s_part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, q = lane >> 4;
  const int e0 = 16 * blockIdx.x, t0 = 16 * blockIdx.y;
  const int e = e0 + row, t = t0 + row;
  const int kw = a.H / (4 * a.S);  // columns per wave
  const size_t c0 = (size_t)blockIdx.z * (a.H / a.S) + (size_t)wave * kw;
  const uint4 *wr = reinterpret_cast<const uint4 *>(a.router + (size_t)(e < a.E ? e : 0) * a.H +
                                                    c0 + 8 * q);
  const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + (size_t)(t < a.T ? t : 0) * a.H +
                                                    c0 + 8 * q);
  const bool ev = e < a.E, tv = t < a.T;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kw / 32; ++k) {
    uint4 av = wr[4 * k], bv = xr[4 * k];
    if (!ev) av = make_uint4(0, 0, 0, 0);
    if (!tv) bv = make_uint4(0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t r = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4_t p = s_part[w][lane];
      r[0] += p[0];
      r[1] += p[1];
      r[2] += p[2];
      r[3] += p[3];
    }
    // element v of lane: expert e0 + 4 q + v, token t0 + row
    if (t0 + row < a.T) {
      float *lp = a.logits + ((size_t)blockIdx.z * a.T + t0 + row) * a.E;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ee = e0 + 4 * q + v;
        if (ee < a.E) lp[ee] = r[v];
      }
    }
  }
}

// Many tokens: a block computes a 64-token x 64-expert tile of the logits
// over one of S column ranges.  The x and router rows of each 64-column step
// are staged in LDS once per block (the 16 x 16 tiles above read each row
// once per tile, which makes a large batch bound by cache traffic); wave w
// computes the 32 x 32 quarter of tokens 32 (w & 1) .. and experts
// 32 (w >> 1) .. of the tile.
// v, or zeros where !ok (per component: a select of the whole struct goes
// through memory)
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

constexpr int kRtTile = 64;  // tokens and experts per block
constexpr int kRtStep = 64;  // columns per staged step

__global__ void __launch_bounds__(256) k_router_tiled(RouteArgs a) {
  constexpr int SEG = kRtStep / 8;  // 16-byte segments per staged row
  constexpr int LD = SEG + 1;       // row pitch in uint4 (+1 against bank conflicts)
  __shared__ uint4 s_x[2][kRtTile * LD];
  __shared__ uint4 s_r[2][kRtTile * LD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, c16 = lane & 15;
  const int t0 = kRtTile * blockIdx.y, e0 = kRtTile * blockIdx.x;
  const int kw = a.H / a.S;
  const size_t kb = (size_t)blockIdx.z * kw;
  const int nst = kw / kRtStep;
  // this thread's two pieces of each operand per step: row p / SEG, segment
  // p % SEG (p = tid, tid + 256); rows past T or E read the tile's first row
  // and stage zeros (the loads are issued on every path)
  const int pr0 = tid / SEG, pr1 = pr0 + 256 / SEG, ps = tid % SEG;
  const bool xok0 = t0 + pr0 < a.T, xok1 = t0 + pr1 < a.T;
  const bool rok0 = e0 + pr0 < a.E, rok1 = e0 + pr1 < a.E;
  const uint4 *xp0 = reinterpret_cast<const uint4 *>(a.x + (size_t)(xok0 ? t0 + pr0 : t0) * a.H + kb) + ps;
  const uint4 *xp1 = reinterpret_cast<const uint4 *>(a.x + (size_t)(xok1 ? t0 + pr1 : t0) * a.H + kb) + ps;
  const uint4 *rp0 = reinterpret_cast<const uint4 *>(a.router + (size_t)(rok0 ? e0 + pr0 : e0) * a.H + kb) + ps;
  const uint4 *rp1 = reinterpret_cast<const uint4 *>(a.router + (size_t)(rok1 ? e0 + pr1 : e0) * a.H + kb) + ps;
  const int so0 = pr0 * LD + ps, so1 = pr1 * LD + ps;
  const int wt = wave & 1, we = wave >> 1;
  f32x4_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 x0 = xp0[0], x1 = xp1[0], r0 = rp0[0], r1 = rp1[0];
  s_x[0][so0] = keep_if(xok0, x0);
  s_x[0][so1] = keep_if(xok1, x1);
  s_r[0][so0] = keep_if(rok0, r0);
  s_r[0][so1] = keep_if(rok1, r1);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) {
      x0 = xp0[(st + 1) * SEG];
      x1 = xp1[(st + 1) * SEG];
      r0 = rp0[(st + 1) * SEG];
      r1 = rp1[(st + 1) * SEG];
    }
    // A operand: token rows (lane: row c16, columns 8 q .. of a 32-column
    // half step); B operand: expert rows, the same columns
#pragma unroll
    for (int kk = 0; kk < kRtStep / 32; ++kk) {
      bf16x8_t av[2], bv[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        av[mi] = __builtin_bit_cast(bf16x8_t, s_x[buf][(32 * wt + 16 * mi + c16) * LD + 4 * kk + q]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bv[ni] = __builtin_bit_cast(bf16x8_t, s_r[buf][(32 * we + 16 * ni + c16) * LD + 4 * kk + q]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
    if (st + 1 < nst) {
      s_x[buf ^ 1][so0] = keep_if(xok0, x0);
      s_x[buf ^ 1][so1] = keep_if(xok1, x1);
      s_r[buf ^ 1][so0] = keep_if(rok0, r0);
      s_r[buf ^ 1][so1] = keep_if(rok1, r1);
    }
    __syncthreads();
  }
  // element v of acc[mi][ni]: token 32 wt + 16 mi + 4 q + v, expert
  // 32 we + 16 ni + c16 of the tile
  float *lp = a.logits + (size_t)blockIdx.z * a.T * a.E;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 32 * wt + 16 * mi + 4 * q + v, e = e0 + 32 * we + 16 * ni + c16;
        if (t < a.T && e < a.E) lp[(size_t)t * a.E + e] = acc[mi][ni][v];
      }
}

// One block per token: the 4 waves add the S partial logits in order (all
// loads in flight at once) into LDS, then wave 0 selects the top-K (largest
// first; equal logits -> lower index) and the weights = softmax over the
// selected logits.
__global__ void __launch_bounds__(256) k_topk(RouteArgs a) {
  __shared__ float s_l[kMaxE];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const float *lt = a.logits + (size_t)t * a.E;
  constexpr int NI = kMaxE / 256;
  float p[NI][kMaxRouteSplits];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = tid + 256 * i;
#pragma unroll
    for (int sp = 0; sp < kMaxRouteSplits; ++sp)
      p[i][sp] = (idx < a.E && sp < a.S) ? lt[(size_t)sp * a.T * a.E + idx] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = tid + 256 * i;
    if (idx < a.E) {
      float v = p[i][0];
#pragma unroll
      for (int sp = 1; sp < kMaxRouteSplits; ++sp)
        if (sp < a.S) v += p[i][sp];
      s_l[idx] = v;
      if (a.logits_out) a.logits_out[(size_t)t * a.E + idx] = v;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  constexpr int NV = kMaxE / 64;
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int idx = lane + 64 * j;
    const float v = idx < a.E ? s_l[idx] : __builtin_nanf("");
    key[j] = ((uint64_t)f32_order_key(v) << 32) | (0xFFFFFFFFu - (uint32_t)idx);
  }
  float sel_v[kMaxK];
  int sel_i[kMaxK];
  for (int k = 0; k < a.K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) best = key[j] > best ? key[j] : best;
    const uint64_t m = wave_max_u64(best);
    const uint32_t k32 = (uint32_t)(m >> 32);
    sel_i[k] = m == 0 ? -1 : (int)(0xFFFFFFFFu - (uint32_t)m);
    sel_v[k] = __uint_as_float((k32 & 0x80000000u) ? (k32 & 0x7FFFFFFFu) : ~k32);
#pragma unroll
    for (int j = 0; j < NV; ++j) key[j] = key[j] == m ? 0 : key[j];
  }
  if (lane == 0) {
    float den = 0.f, pk[kMaxK];
    for (int k = 0; k < a.K; ++k) {
      pk[k] = expf(sel_v[k] - sel_v[0]);
      den += pk[k];
    }
    for (int k = 0; k < a.K; ++k) {
      a.ids[(size_t)t * a.K + k] = sel_i[k];
      a.w[(size_t)t * a.K + k] = pk[k] / den;
    }
  }
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU.  Block = (token, slot, block of rows).  Each wave covers
// kLoadsGU wave-wide loads of gate and up rows (rpl rows per load).
// ---------------------------------------------------------------------------
constexpr int kLoadsGU = 2;
constexpr int kLoadsDown = 2;

struct GateUpArgs {
  const uint16_t *x;
  const uint8_t *experts, *shared;
  int64_t stride;
  const int32_t *ids;
  float *h;
  Ctrl *ctrl;
  int H, I, E, K, slots, T;
  int64_t off_gq, off_uq, off_gsb, off_usb;
  RowGeo geo;
  int rows_per_block, blocks_per_slot;
};

template <int BITS>
__global__ void __launch_bounds__(256) k_gateup(GateUpArgs a) {
  extern __shared__ uint32_t smem[];
  constexpr int kPairs = XSeg<BITS>::kPairs;
  const int nseg_row = a.geo.seg_per_row;
  uint32_t *xp = smem;
  float2 *cx = reinterpret_cast<float2 *>(smem + nseg_row * kPairs);

  const int rb = blockIdx.x % a.blocks_per_slot;
  const int slot = (blockIdx.x / a.blocks_per_slot) % a.slots;
  const int t = blockIdx.x / (a.blocks_per_slot * a.slots);

  const uint8_t *blob;
  if (slot < a.K) {
    const int e = a.ids[(size_t)t * a.K + slot];
    if (e < 0 || e >= a.E) {
      // invalid id: this slot contributes nothing
      const int r = rb * a.rows_per_block + threadIdx.x;
      if (threadIdx.x < a.rows_per_block)
        a.h[((size_t)t * a.slots + slot) * a.I + r] = 0.f;
      if (threadIdx.x == 0) atomicOr(&a.ctrl->err, 1u);
      return;
    }
    blob = a.experts + (size_t)e * a.stride;
  } else {
    blob = a.shared;
  }

  stage_x<BITS>(a.x + (size_t)t * a.H, a.H, xp, cx);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lpr = a.geo.lpr, rpl = a.geo.rpl;
  const int sl = lane % lpr;
  const size_t row_bytes = (size_t)nseg_row * 16;
  const int groups = a.H / kGroup;
  const uint8_t *gq = blob + a.off_gq, *uq = blob + a.off_uq;
  const uint32_t *gsb = reinterpret_cast<const uint32_t *>(blob + a.off_gsb);
  const uint32_t *usb = reinterpret_cast<const uint32_t *>(blob + a.off_usb);
  const int row0 = rb * a.rows_per_block + wave * (kLoadsGU * rpl);

#pragma unroll
  for (int ld = 0; ld < kLoadsGU; ++ld) {
    const int r = row0 + ld * rpl + lane / lpr;
    float pg = 0.f, pu = 0.f;
    for (int k = 0; k < a.geo.nseg; ++k) {
      const int sg = sl + k * lpr;
      const uint4 cg = ldg16(gq + r * row_bytes + (size_t)sg * 16);
      const uint4 cu = ldg16(uq + r * row_bytes + (size_t)sg * 16);
      const int grp = sg * XSeg<BITS>::kCols / kGroup;
      const uint32_t sbg = gsb[(size_t)r * groups + grp];
      const uint32_t sbu = usb[(size_t)r * groups + grp];
      const uint32_t *xs = xp + sg * kPairs;
      const float2 c = cx[sg];
      const float ag = seg_dot_x<BITS>(cg, xs) - c.x;
      const float au = seg_dot_x<BITS>(cu, xs) - c.x;
      pg += bf16f(sbg & 0xFFFFu) * ag + bf16f(sbg >> 16) * c.y;
      pu += bf16f(sbu & 0xFFFFu) * au + bf16f(sbu >> 16) * c.y;
    }
    pg = group_sum(pg, lpr);
    pu = group_sum(pu, lpr);
    if (sl == 0) {
      const float hv = pg / (1.f + expf(-pg)) * pu;
      a.h[((size_t)t * a.slots + slot) * a.I + r] = hv;
    }
  }
}

// ---------------------------------------------------------------------------
// Down + combine.  Block = (token, block of output rows); it walks the slots
// in order (routed experts in rank order, then the shared expert), staging
// each slot's activations in LDS, and accumulates w_k * (Down_k h_k) per row.
// ---------------------------------------------------------------------------
struct DownArgs {
  const uint8_t *experts, *shared;
  int64_t stride;
  const int32_t *ids;
  const float *w;
  const float *h;
  float *y;
  Ctrl *ctrl;
  int H, I, E, K, slots, T;
  int64_t off_dq, off_dsb;
  RowGeo geo;
  int rows_per_block, blocks_per_token;
};

template <int BITS>
__global__ void __launch_bounds__(256) k_down(DownArgs a) {
  extern __shared__ uint32_t smem[];
  constexpr int kPairs = XSeg<BITS>::kPairs;
  const int nseg_row = a.geo.seg_per_row;
  uint32_t *hp = smem;
  float2 *cx = reinterpret_cast<float2 *>(smem + nseg_row * 2 * kPairs);

  const int rb = blockIdx.x % a.blocks_per_token;
  const int t = blockIdx.x / a.blocks_per_token;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lpr = a.geo.lpr, rpl = a.geo.rpl;
  const int sl = lane % lpr;
  const size_t row_bytes = (size_t)nseg_row * 16;
  const int groups = a.I / kGroup;
  const int row0 = rb * a.rows_per_block + wave * (kLoadsDown * rpl);

  float acc[kLoadsDown];
#pragma unroll
  for (int ld = 0; ld < kLoadsDown; ++ld) acc[ld] = 0.f;

  for (int slot = 0; slot < a.slots; ++slot) {
    const uint8_t *blob;
    float wk;
    if (slot < a.K) {
      const int e = a.ids[(size_t)t * a.K + slot];
      if (e < 0 || e >= a.E) continue;  // uniform across the block
      blob = a.experts + (size_t)e * a.stride;
      wk = a.w[(size_t)t * a.K + slot];
    } else {
      blob = a.shared;
      wk = 1.f;
    }
    __syncthreads();
    stage_h<BITS>(a.h + ((size_t)t * a.slots + slot) * a.I, a.I, hp, cx);
    __syncthreads();
    const uint8_t *dq = blob + a.off_dq;
    const uint32_t *dsb = reinterpret_cast<const uint32_t *>(blob + a.off_dsb);
#pragma unroll
    for (int ld = 0; ld < kLoadsDown; ++ld) {
      const int r = row0 + ld * rpl + lane / lpr;
      float p = 0.f;
      for (int k = 0; k < a.geo.nseg; ++k) {
        const int sg = sl + k * lpr;
        const uint4 c = ldg16(dq + r * row_bytes + (size_t)sg * 16);
        const uint32_t sb = dsb[(size_t)r * groups + sg * XSeg<BITS>::kCols / kGroup];
        const float2 cc = cx[sg];
        const float q = seg_dot_h<BITS>(c, hp + sg * 2 * kPairs) - cc.x;
        p += bf16f(sb & 0xFFFFu) * q + bf16f(sb >> 16) * cc.y;
      }
      acc[ld] += wk * p;
    }
  }
#pragma unroll
  for (int ld = 0; ld < kLoadsDown; ++ld) {
    const float v = group_sum(acc[ld], lpr);
    const int r = row0 + ld * rpl + lane / lpr;
    if (sl == 0) a.y[(size_t)t * a.H + r] = v;
  }
}

// ---------------------------------------------------------------------------
// Dequantisation hooks: one thread per code word; each writes s q + z for
// the word's codes, with q as the named decoder produces it.
//   k_dequantize        mask and shift per code (the plain reading of the format)
//   k_dequant_pairs<1>  fp16 pairs 1024 + m q (h2_code_pair: single-token and
//                       unfused gate/up products)
//   k_dequant_pairs<3>  bf16 pairs 128 + q (b2_code_pair: unfused down products)
// The fp8 pair convert of the single-token down products and the bf16 slices
// of the grouped GEMM have their hooks beside their kernels.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_dequantize(DequantArgs a) {
  const int cpw = 32 / a.bits;
  const int wpr = a.cols / cpw;
  const size_t n = (size_t)a.rows * wpr;
  const uint32_t mask = (1u << a.bits) - 1u;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const int c0 = (int)(i - r * wpr) * cpw;
    const uint32_t w = a.q[i];
    const uint32_t sz = a.sb[r * (a.cols / kGroup) + c0 / kGroup];
    const float s = bf16f(sz & 0xFFFFu), z = bf16f(sz >> 16);
    float *o = a.out + r * a.cols + c0;
    for (int j = 0; j < cpw; ++j) o[j] = fmaf(s, (float)((w >> (a.bits * j)) & mask), z);
  }
}

template <int BITS, int DEC>
__global__ void __launch_bounds__(256) k_dequant_pairs(DequantArgs a) {
  constexpr int CPW = 32 / BITS, NP = CPW / 2;
  const int wpr = a.cols / CPW;
  const size_t n = (size_t)a.rows * wpr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const int c0 = (int)(i - r * wpr) * CPW;
    const uint32_t w = a.q[i];
    float q[CPW];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // pair p holds codes (p, p + NP) of the word
      if (DEC == MOE_DEQ_FP16_PAIR) {
        const uint32_t v = h2_code_pair<BITS>(w, h2_shifted<BITS>(w), p);
        const h2_t hv = __builtin_bit_cast(h2_t, v);
        // 1024 + m q with m = 16^(p & 1) (4 bits) or 4^f (2 bits); 1 / m is exact
        const int f = BITS == 4 ? 2 * (p & 1) : (p < 5 ? p : p - 5);
        const float im = 1.f / (float)(1 << (2 * f));
        q[p] = ((float)hv.x - 1024.f) * im;
        q[p + NP] = ((float)hv.y - 1024.f) * im;
      } else {
        const uint32_t v = b2_code_pair<BITS>(w, p);
        q[p] = bf16f(v & 0xFFFFu) - 128.f;
        q[p + NP] = bf16f(v >> 16) - 128.f;
      }
    }
    store_dequant_word<CPW>(a, r, c0, q);
  }
}

// ---------------------------------------------------------------------------
// Residual stream around the layer, for the multi-token and unfused paths.
// x[t] = bf16(r[t] / sqrt(mean_c r[t][c]^2 + eps)), one workgroup per token;
// the sum of squares is reduced in a fixed order (deterministic).
// ---------------------------------------------------------------------------
constexpr float kRmsEps = 1e-6f;

__global__ void __launch_bounds__(256) k_rmsnorm(const float *__restrict__ r, int H,
                                                 uint16_t *__restrict__ x) {
  __shared__ float s_part[4];
  const float *rt = r + (size_t)blockIdx.x * H;
  uint16_t *xt = x + (size_t)blockIdx.x * H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  for (int c = 4 * threadIdx.x; c < H; c += 1024) {
    const float4 v = *reinterpret_cast<const float4 *>(rt + c);
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum64(ss);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  const float tot = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  const float inv = 1.f / sqrtf(tot * (1.f / (float)H) + kRmsEps);
  for (int c = 4 * threadIdx.x; c < H; c += 1024) {
    const float4 v = *reinterpret_cast<const float4 *>(rt + c);
    *reinterpret_cast<uint2 *>(xt + c) =
        make_uint2(f2bf(v.x * inv) | (f2bf(v.y * inv) << 16), f2bf(v.z * inv) | (f2bf(v.w * inv) << 16));
  }
}

// r += y over n floats (n a multiple of 4).
__global__ void __launch_bounds__(256) k_resid_add(float *__restrict__ r,
                                                   const float *__restrict__ y, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    float4 a = reinterpret_cast<float4 *>(r)[i];
    const float4 b = reinterpret_cast<const float4 *>(y)[i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
    reinterpret_cast<float4 *>(r)[i] = a;
  }
}

__global__ void k_ws_init(uint4 *ctrl, int n16) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
    ctrl[i] = make_uint4(0u, 0u, 0u, 0u);
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Allows `bytes` of dynamic LDS for kernel f (the default cap is 64 KB).
template <typename F>
int allow_lds(F f, size_t bytes) {
  if (bytes > kMaxLds) return (int)hipErrorInvalidValue;
  if (bytes <= 64 * 1024) return 0;
  return (int)hipFuncSetAttribute(reinterpret_cast<const void *>(f),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_ws_init(void *ws, size_t, void *stream) {
  static_assert(kHeaderBytes % 16 == 0, "header is a multiple of 16 bytes");
  hipLaunchKernelGGL(k_ws_init, dim3(64), dim3(256), 0, S(stream), static_cast<uint4 *>(ws),
                     (int)(kHeaderBytes / 16));
  return (int)hipGetLastError();
}

int launch_route(const moe_dims &d, const uint16_t *router, const uint16_t *x, int T,
                 int32_t *ids, float *w, float *logits, void *ws, void *stream) {
  const WsLayout W = ws_layout(d, T);
  uint8_t *base = static_cast<uint8_t *>(ws);
  RouteArgs a;
  a.router = router;
  a.x = x;
  a.ids = ids;
  a.w = w;
  a.logits_out = logits;
  a.logits = reinterpret_cast<float *>(base + W.logits);
  a.H = d.hidden;
  a.E = d.n_experts;
  a.K = d.top_k;
  a.T = T;
  a.S = route_splits(d, T);
  if (route_tiled(T))
    hipLaunchKernelGGL(k_router_tiled,
                       dim3((d.n_experts + kRtTile - 1) / kRtTile, (T + kRtTile - 1) / kRtTile, a.S),
                       dim3(256), 0, S(stream), a);
  else
    hipLaunchKernelGGL(k_router, dim3((d.n_experts + 15) / 16, (T + 15) / 16, a.S), dim3(256), 0,
                       S(stream), a);
  hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, S(stream), a);
  return (int)hipGetLastError();
}

int launch_expert_forward(const moe_dims &d, const moe_layer &L, const uint16_t *x, int T,
                          const int32_t *ids, const float *w, float *y, void *ws,
                          void *stream) {
  const WsLayout W = ws_layout(d, T);
  const BlobLayout B = blob_layout(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  float *h = reinterpret_cast<float *>(base + W.h);
  Ctrl *ctrl = reinterpret_cast<Ctrl *>(base + W.ctrl);
  const int slots = d.top_k + d.has_shared;
  const int pairs = 64 / d.bits;  // packed pairs per 16-byte segment

  GateUpArgs g;
  g.x = x;
  g.experts = L.experts;
  g.shared = L.shared;
  g.stride = L.expert_stride;
  g.ids = ids;
  g.h = h;
  g.ctrl = ctrl;
  g.H = d.hidden;
  g.I = d.inter;
  g.E = d.n_experts;
  g.K = d.top_k;
  g.slots = slots;
  g.T = T;
  g.off_gq = (int64_t)B.off[MOE_SEC_GATE_Q];
  g.off_uq = (int64_t)B.off[MOE_SEC_UP_Q];
  g.off_gsb = (int64_t)B.off[MOE_SEC_GATE_SB];
  g.off_usb = (int64_t)B.off[MOE_SEC_UP_SB];
  g.geo = row_geo(d.hidden, d.bits);
  g.rows_per_block = 4 * kLoadsGU * g.geo.rpl;
  if (g.rows_per_block > d.inter) return (int)hipErrorInvalidValue;
  g.blocks_per_slot = d.inter / g.rows_per_block;
  const size_t lds_gu = (size_t)g.geo.seg_per_row * (pairs * 4 + 8);
  const dim3 grid_gu((unsigned)(g.blocks_per_slot * slots * T));

  DownArgs dn;
  dn.experts = L.experts;
  dn.shared = L.shared;
  dn.stride = L.expert_stride;
  dn.ids = ids;
  dn.w = w;
  dn.h = h;
  dn.y = y;
  dn.ctrl = ctrl;
  dn.H = d.hidden;
  dn.I = d.inter;
  dn.E = d.n_experts;
  dn.K = d.top_k;
  dn.slots = slots;
  dn.T = T;
  dn.off_dq = (int64_t)B.off[MOE_SEC_DOWN_Q];
  dn.off_dsb = (int64_t)B.off[MOE_SEC_DOWN_SB];
  dn.geo = row_geo(d.inter, d.bits);
  dn.rows_per_block = 4 * kLoadsDown * dn.geo.rpl;
  if (dn.rows_per_block > d.hidden) return (int)hipErrorInvalidValue;
  dn.blocks_per_token = d.hidden / dn.rows_per_block;
  const size_t lds_dn = (size_t)dn.geo.seg_per_row * (2 * pairs * 4 + 8);
  const dim3 grid_dn((unsigned)(dn.blocks_per_token * T));

  if (d.bits == 4) {
    if (allow_lds(k_gateup<4>, lds_gu) || allow_lds(k_down<4>, lds_dn))
      return (int)hipErrorInvalidValue;
    timing::mark(MOE_ST_GATEUP);
    hipLaunchKernelGGL(k_gateup<4>, grid_gu, dim3(256), lds_gu, S(stream), g);
    timing::mark(MOE_ST_DOWN);
    hipLaunchKernelGGL(k_down<4>, grid_dn, dim3(256), lds_dn, S(stream), dn);
  } else {
    if (allow_lds(k_gateup<2>, lds_gu) || allow_lds(k_down<2>, lds_dn))
      return (int)hipErrorInvalidValue;
    timing::mark(MOE_ST_GATEUP);
    hipLaunchKernelGGL(k_gateup<2>, grid_gu, dim3(256), lds_gu, S(stream), g);
    timing::mark(MOE_ST_DOWN);
    hipLaunchKernelGGL(k_down<2>, grid_dn, dim3(256), lds_dn, S(stream), dn);
  }
  return (int)hipGetLastError();
}

int launch_rmsnorm(const moe_dims &d, const float *r, int T, uint16_t *x, void *stream) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, S(stream), r, d.hidden, x);
  return (int)hipGetLastError();
}

int launch_resid_add(const moe_dims &d, float *r, const float *y, int T, void *stream) {
  const size_t n4 = (size_t)T * d.hidden / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_resid_add, dim3((unsigned)blocks), dim3(256), 0, S(stream), r, y, n4);
  return (int)hipGetLastError();
}

int launch_dequantize_as(const moe_dims &d, const uint8_t *blob, int which, int decoder,
                         float *out, void *stream) {
  const BlobLayout B = blob_layout(d);
  DequantArgs a;
  a.q = reinterpret_cast<const uint32_t *>(blob + B.off[which]);
  a.sb = reinterpret_cast<const uint32_t *>(blob + B.off[3 + which]);
  a.out = out;
  a.rows = which == 2 ? d.hidden : d.inter;
  a.cols = which == 2 ? d.inter : d.hidden;
  a.bits = d.bits;
  const size_t words = (size_t)a.rows * a.cols / (32 / d.bits);
  size_t blocks = (words + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 g((unsigned)blocks), b(256);
  switch (decoder) {
    case MOE_DEQ_SCALAR:
      hipLaunchKernelGGL(k_dequantize, g, b, 0, S(stream), a);
      break;
    case MOE_DEQ_FP16_PAIR:
      if (d.bits == 4) hipLaunchKernelGGL((k_dequant_pairs<4, MOE_DEQ_FP16_PAIR>), g, b, 0, S(stream), a);
      else hipLaunchKernelGGL((k_dequant_pairs<2, MOE_DEQ_FP16_PAIR>), g, b, 0, S(stream), a);
      break;
    case MOE_DEQ_BF16_PAIR:
      if (d.bits == 4) hipLaunchKernelGGL((k_dequant_pairs<4, MOE_DEQ_BF16_PAIR>), g, b, 0, S(stream), a);
      else hipLaunchKernelGGL((k_dequant_pairs<2, MOE_DEQ_BF16_PAIR>), g, b, 0, S(stream), a);
      break;
    case MOE_DEQ_FP8_PAIR:
      return launch_dequant_fp8(a, (int)blocks, stream);
    case MOE_DEQ_BF16_SLICE:
      return launch_dequant_slices(a, (int)blocks, stream);
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int read_device_error(void *ws, void *stream, int32_t *err) {
  Ctrl *ctrl = static_cast<Ctrl *>(ws);
  hipError_t e = hipStreamSynchronize(S(stream));
  if (e != hipSuccess) return (int)e;
  uint32_t v = 0;
  e = hipMemcpy(&v, &ctrl->err, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  const uint32_t zero = 0;
  e = hipMemcpy(&ctrl->err, &zero, 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) return (int)e;
  *err = (int32_t)v;
  return 0;
}

}  // namespace moe
