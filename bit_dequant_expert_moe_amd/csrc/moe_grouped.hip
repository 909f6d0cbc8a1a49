// moe_grouped.hip -- the MoE layer for a batch of T >= 2 tokens.
//
// Method: "Flash-MoE: Running a 397B Parameter Model on a Laptop"
// (hysenlabs.com), section "How the SSD expert streaming pipeline works":
// per token, router -> softmax + top-K -> forward pass of the selected
// experts and the shared expert -> combine.  For several tokens at once the
// (token, slot) pairs are grouped by expert first, so that every selected
// expert's weights are read once for all tokens routed to it and the shared
// expert once for the whole batch.
//
// Kernels
//   k_bucket     counting sort of the T*K (token, slot) pairs by expert:
//                bucket list (routed experts in increasing id, then the shared
//                expert with all T tokens), offsets and pair codes.
//   k_grouped    dequantising grouped GEMM on the matrix cores for one
//                (bucket, 64-row tile, 32-pair chunk):
//                  gate/up: h = silu(Gate x) * (Up x) for every pair;
//                  down:    yd = Down h for every pair.
//   k_combine    y[t] = sum_k w[t][k] yd[t][k] + yd[t][shared], in that order.
//
// Matrix-core arithmetic.  A group of 64 weights of a row shares (s, z), so
//   sum_c (s q_c + z) b_c = s * sum_c q_c b_c + z * sum_c b_c.
// The codes enter v_mfma_f32_16x16x32_bf16 as bf16 values 128 + q (exact: one
// v_and_or_b32 puts two 4-bit fields into the mantissas of a pair of bf16
// 128.0); the product with the bf16 activations is exact and the MFMA sums in
// fp32.  Per group the partial result P gives sum q b = P - 128 * sum b, which
// is scaled and biased in fp32.  x is bf16 already; h (fp32) enters as
// bf16 hi + bf16 lo, two MFMAs, ~16 significant bits.
//
// The field order inside a code word makes the A operand of a lane hold the
// columns (c0, c4, c1, c5, c2, c6, c3, c7) of its 8-column slice; the staged
// B operand uses the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRT = 64;         // weight rows per block (16 per wave)
constexpr int kNC = 32;         // pairs per block (two 16-wide MFMA tiles)
constexpr int kKC = 256;        // columns per staged chunk
constexpr int kGC = kKC / kGroup;  // groups per chunk (4)
constexpr int kSl = kKC / 8;    // 8-column slices per chunk (32)

// ---------------------------------------------------------------------------
// Buckets.  Layout of the int32 array bk (maxB = min(E, T K) + has_shared):
//   bk[0]                       number of buckets nb
//   bk[1 + j]                   expert of bucket j (E = the shared expert)
//   bk[1 + maxB + j], j <= nb   first pair of bucket j; bk[1 + maxB + nb] = total
//   bk[2 + 2 maxB + p]          pair code t (K + 1) + slot (slot K = shared)
// ---------------------------------------------------------------------------
struct BucketArgs {
  const int32_t *ids;
  int32_t *bk;
  Ctrl *ctrl;
  int T, K, E, has_shared, maxB;
};

// Exclusive prefix sum over the 1024 threads of the block; returns the sum of
// the values of the lower threads and writes the block total to *total.
__device__ int block_exscan(int v, int *wtot, int *total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  if (w == 0) {
    int t = lane < 16 ? wtot[lane] : 0;
    int ti = t;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(ti, d, 64);
      if (lane >= d) ti += o;
    }
    if (lane < 16) wtot[lane] = ti - t;  // exclusive per wave
    if (lane == 15) wtot[16] = ti;
  }
  __syncthreads();
  const int r = wtot[w] + inc - v;
  *total = wtot[16];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024) k_bucket(BucketArgs a) {
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_pos[kMaxE];
  __shared__ int s_wtot[17];
  const int tid = threadIdx.x;
  const int np = a.T * a.K;
  for (int e = tid; e < kMaxE; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < np; p += 1024) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.E) atomicAdd(&s_cnt[e], 1);
    else atomicOr(&a.ctrl->err, 1u);  // that slot contributes nothing
  }
  __syncthreads();
  // one thread per expert (E <= 1024): bucket index and first pair
  const int c = tid < a.E ? s_cnt[tid] : 0;
  int nrb, total;
  const int j = block_exscan(c > 0 ? 1 : 0, s_wtot, &nrb);
  const int off = block_exscan(c, s_wtot, &total);
  int32_t *bexp = a.bk + 1, *boff = a.bk + 1 + a.maxB, *pairs = a.bk + 2 + 2 * a.maxB;
  if (c > 0) {
    bexp[j] = tid;
    boff[j] = off;
    s_pos[tid] = off;
  }
  const int nb = nrb + (a.has_shared ? 1 : 0);
  if (tid == 0) {
    a.bk[0] = nb;
    if (a.has_shared) {
      bexp[nrb] = a.E;
      boff[nrb] = total;
    }
    boff[nb] = total + (a.has_shared ? a.T : 0);
  }
  if (a.has_shared)
    for (int t = tid; t < a.T; t += 1024) pairs[total + t] = t * (a.K + 1) + a.K;
  __syncthreads();
  // the order of pairs inside a bucket does not change any result: each
  // pair's column of the MFMA tiles is computed independently
  for (int p = tid; p < np; p += 1024) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.E) {
      const int at = atomicAdd(&s_pos[e], 1);
      pairs[at] = (p / a.K) * (a.K + 1) + (p % a.K);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped dequantising GEMM.
// ---------------------------------------------------------------------------
struct GroupArgs {
  const uint16_t *x;  // [T][H] bf16 (gate/up)
  const float *hin;   // [T (K+1)][I] fp32 (down)
  const uint8_t *experts, *shared;
  int64_t stride;
  const int32_t *bk;
  float *out;         // gate/up: h [T (K+1)][I]; down: yd [T (K+1)][H]
  int R, C;           // rows and columns of the matrices of this pass
  int E, maxB, K1;    // K1 = K + 1 (pair code = token K1 + slot)
  int64_t off_q0, off_q1, off_sb0, off_sb1;  // second matrix unused for down
};

template <int BITS, bool DOWN>
struct GL {  // LDS geometry
  static constexpr int NMAT = DOWN ? 1 : 2;
  static constexpr int RW = kKC * BITS / 32 + 2;  // words per staged row (+2 against bank conflicts)
  static constexpr int BV = DOWN ? 8 : 4;         // u32 per (pair, slice): bf16x8 (x) or hi + lo
  static constexpr int TS = kSl * BV + 4;         // u32 per staged pair (+4 against bank conflicts)
  static constexpr int A_U32 = NMAT * kRT * RW;
  static constexpr int B_U32 = kNC * TS;
  static constexpr int SB_U32 = NMAT * kRT * kGC;
  static constexpr int XS_F32 = kNC * kGC;
  static constexpr int BUF_U32 = A_U32 + B_U32 + SB_U32 + XS_F32;
  static constexpr size_t BYTES = 2 * (size_t)BUF_U32 * 4;
  static constexpr int PPR = kKC * BITS / 128;    // 16-byte pieces per staged row
  static_assert((kRT * PPR) % 256 == 0 || kRT * PPR == 256, "A pieces tile the block");
};

// Two bf16 (hi half, lo half) of 128 + the fields selected by mask m.
__device__ __forceinline__ uint32_t magic_pair(uint32_t v, uint32_t m) {
  return and_or(v, m, 0x43004300u);
}

// A operand of one 8-column slice: bf16 128 + q in the order
// (c0, c4, c1, c5, c2, c6, c3, c7).  For 2-bit codes the slice is one half
// (16 bits) of a word.
template <int BITS>
__device__ __forceinline__ bf16x8 a_slice(uint32_t word, int half) {
  uint32_t p[4];
  if (BITS == 4) {
    p[0] = magic_pair(word, 0x000F000Fu);
    p[1] = magic_pair(word >> 4, 0x000F000Fu);
    p[2] = magic_pair(word >> 8, 0x000F000Fu);
    p[3] = magic_pair(word >> 12, 0x000F000Fu);
  } else {
    const uint32_t h16 = half ? (word >> 16) : (word & 0xFFFFu);
    const uint32_t v = h16 | (h16 << 8);  // c_{j+4} lands 16 bits above c_j
    p[0] = magic_pair(v, 0x00030003u);
    p[1] = magic_pair(v >> 2, 0x00030003u);
    p[2] = magic_pair(v >> 4, 0x00030003u);
    p[3] = magic_pair(v >> 6, 0x00030003u);
  }
  uint4 u = make_uint4(p[0], p[1], p[2], p[3]);
  return __builtin_bit_cast(bf16x8, u);
}

// (x0..x7 as pairs (x0,x1),(x2,x3),(x4,x5),(x6,x7)) -> (x0,x4),(x1,x5),(x2,x6),(x3,x7)
__device__ __forceinline__ uint4 b_order(uint4 q) {
  uint4 r;
  r.x = (q.x & 0xFFFFu) | (q.z << 16);
  r.y = (q.x >> 16) | (q.z & 0xFFFF0000u);
  r.z = (q.y & 0xFFFFu) | (q.w << 16);
  r.w = (q.y >> 16) | (q.w & 0xFFFF0000u);
  return r;
}

template <int BITS, bool DOWN>
__global__ void __launch_bounds__(256) k_grouped(GroupArgs a) {
  using G = GL<BITS, DOWN>;
  extern __shared__ __align__(16) uint32_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, col = lane & 15;
  const int nb = a.bk[0];
  const int j = blockIdx.y;
  if (j >= nb) return;
  const int e = a.bk[1 + j];
  const int p0 = a.bk[1 + a.maxB + j], p1 = a.bk[2 + a.maxB + j];
  const int pbase = p0 + kNC * (int)blockIdx.z;
  if (pbase >= p1) return;
  const int nn = min(kNC, p1 - pbase);
  const int ntiles = (nn + 15) >> 4;
  const int32_t *pairs = a.bk + 2 + 2 * a.maxB + pbase;
  const uint8_t *blob = e == a.E ? a.shared : a.experts + (size_t)e * a.stride;
  const int row0 = kRT * (int)blockIdx.x;
  const size_t rbytes = (size_t)a.C * BITS / 8;
  const int groups = a.C / kGroup;
  const int nchunks = a.C / kKC;

  // ---- staging of chunk c into buffer buf --------------------------------
  constexpr int APT = G::NMAT * kRT * G::PPR / 256;  // 16-byte A pieces per thread
  uint4 ra[APT > 0 ? APT : 1];
  uint4 rsb = make_uint4(0, 0, 0, 0);
  constexpr int BLD = DOWN ? 8 : 4;  // 16-byte B loads per thread
  uint4 rb[BLD];
  const int bj = tid >> 3, bs = (tid & 7) * 4;  // B: pair bj, slices bs .. bs+3
  const int bcode = bj < nn ? pairs[bj] : 0;
  const int brow = DOWN ? bcode : bcode / a.K1;  // row of hin (pair) or of x (token)

  auto load_chunk = [&](int c) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int pc = tid + 256 * i;
      const int mat = pc / (kRT * G::PPR), rr = (pc / G::PPR) % kRT, c16 = pc % G::PPR;
      const int64_t off = mat ? a.off_q1 : a.off_q0;
      ra[i] = *reinterpret_cast<const uint4 *>(blob + off + (size_t)(row0 + rr) * rbytes +
                                              (size_t)c * (kKC * BITS / 8) + c16 * 16);
    }
    if (tid < G::NMAT * kRT) {
      const int mat = tid / kRT, rr = tid % kRT;
      const int64_t off = mat ? a.off_sb1 : a.off_sb0;
      rsb = *reinterpret_cast<const uint4 *>(blob + off +
                                            ((size_t)(row0 + rr) * groups + (size_t)c * kGC) * 4);
    }
    if (bj < nn) {
#pragma unroll
      for (int i = 0; i < BLD; ++i) {
        if (DOWN) {
          // 4 slices x 8 fp32 of h
          rb[i] = *reinterpret_cast<const uint4 *>(a.hin + (size_t)brow * a.C + (size_t)c * kKC +
                                                  (size_t)bs * 8 + 4 * i);
        } else {
          rb[i] = *reinterpret_cast<const uint4 *>(a.x + (size_t)brow * a.C + (size_t)c * kKC +
                                                  (size_t)(bs + i) * 8);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < BLD; ++i) rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_chunk = [&](int buf) {
    uint32_t *A = lds + (size_t)buf * G::BUF_U32;
    uint32_t *B = A + G::A_U32;
    uint32_t *SB = B + G::B_U32;
    float *XS = reinterpret_cast<float *>(SB + G::SB_U32);
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int pc = tid + 256 * i;
      const int mat = pc / (kRT * G::PPR), rr = (pc / G::PPR) % kRT, c16 = pc % G::PPR;
      uint32_t *dst = A + (mat * kRT + rr) * G::RW + c16 * 4;
      dst[0] = ra[i].x;
      dst[1] = ra[i].y;
      dst[2] = ra[i].z;
      dst[3] = ra[i].w;
    }
    if (tid < G::NMAT * kRT) *reinterpret_cast<uint4 *>(SB + tid * kGC) = rsb;
    float part = 0.f;
    if (!DOWN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = rb[i];
        part += bf16f(v.x & 0xFFFFu) + bf16f(v.x >> 16) + bf16f(v.y & 0xFFFFu) + bf16f(v.y >> 16) +
                bf16f(v.z & 0xFFFFu) + bf16f(v.z >> 16) + bf16f(v.w & 0xFFFFu) + bf16f(v.w >> 16);
        *reinterpret_cast<uint4 *>(B + bj * G::TS + (bs + i) * G::BV) = b_order(v);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f[8] = {__uint_as_float(rb[2 * i].x), __uint_as_float(rb[2 * i].y),
                            __uint_as_float(rb[2 * i].z), __uint_as_float(rb[2 * i].w),
                            __uint_as_float(rb[2 * i + 1].x), __uint_as_float(rb[2 * i + 1].y),
                            __uint_as_float(rb[2 * i + 1].z), __uint_as_float(rb[2 * i + 1].w)};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          hi[k] = f2bf(f[k]);
          const float r = f[k] - bf16f(hi[k]);
          lo[k] = f2bf(r);
          part += bf16f(hi[k]) + bf16f(lo[k]);
        }
        const uint4 vh = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                    hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
        const uint4 vl = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                    lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
        uint32_t *dst = B + bj * G::TS + (bs + i) * G::BV;
        *reinterpret_cast<uint4 *>(dst) = b_order(vh);
        *reinterpret_cast<uint4 *>(dst + 4) = b_order(vl);
      }
    }
    // a group is 8 slices = this thread's 4 and its neighbour's
    part += __shfl_xor(part, 1, 64);
    if ((tid & 1) == 0) XS[bj * kGC + (bs >> 3)] = part;
  };

  // ---- accumulators: [matrix][tile][4 rows] --------------------------------
  f32x4 acc[G::NMAT][2];
#pragma unroll
  for (int m = 0; m < G::NMAT; ++m)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ar = wave * 16 + col;  // A row of this lane within the tile
  auto compute_chunk = [&](int buf) {
    const uint32_t *A = lds + (size_t)buf * G::BUF_U32;
    const uint32_t *B = A + G::A_U32;
    const uint32_t *SB = B + G::B_U32;
    const float *XS = reinterpret_cast<const float *>(SB + G::SB_U32);
#pragma unroll
    for (int gi = 0; gi < kGC; ++gi) {
      bf16x8 av[G::NMAT][2];
#pragma unroll
      for (int m = 0; m < G::NMAT; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int sl = 8 * gi + 4 * h + q;  // slice of this lane
          const uint32_t w = A[(m * kRT + ar) * G::RW + (BITS == 4 ? sl : (sl >> 1))];
          av[m][h] = a_slice<BITS>(w, sl & 1);
        }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t >= ntiles) break;
        const int bp = 16 * t + col;  // pair of this lane's B column
        f32x4 P[G::NMAT];
#pragma unroll
        for (int m = 0; m < G::NMAT; ++m) P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int sl = 8 * gi + 4 * h + q;
          const uint32_t *src = B + bp * G::TS + sl * G::BV;
          const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src));
#pragma unroll
          for (int m = 0; m < G::NMAT; ++m)
            P[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][h], bv, P[m], 0, 0, 0);
          if (DOWN) {
            const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src + 4));
#pragma unroll
            for (int m = 0; m < G::NMAT; ++m)
              P[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][h], bl, P[m], 0, 0, 0);
          }
        }
        // output element v of this lane: row 4 q + v of the wave's 16, pair bp
        const float X = XS[bp * kGC + gi];
#pragma unroll
        for (int m = 0; m < G::NMAT; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t sb = SB[(m * kRT + wave * 16 + 4 * q + v) * kGC + gi];
            acc[m][t][v] += bf16f(sb & 0xFFFFu) * (P[m][v] - 128.f * X) + bf16f(sb >> 16) * X;
          }
      }
    }
  };

  // ---- software pipeline over the column chunks ----------------------------
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load_chunk(c + 1);
    compute_chunk(buf);
    if (c + 1 < nchunks) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bp = 16 * t + col;
    if (t < ntiles && bp < nn) {
      const int code = pairs[bp];
      float4 o;
      float *ov = reinterpret_cast<float *>(&o);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (DOWN) {
          ov[v] = acc[0][t][v];
        } else {
          const float g = acc[0][t][v], u = acc[G::NMAT - 1][t][v];
          ov[v] = g / (1.f + expf(-g)) * u;
        }
      }
      *reinterpret_cast<float4 *>(a.out + (size_t)code * a.R + row0 + wave * 16 + 4 * q) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t][r] = sum_{k<K} w[t][k] yd[t(K+1)+k][r] + yd[t(K+1)+K][r].
// ---------------------------------------------------------------------------
struct CombineArgs {
  const float *yd;
  const int32_t *ids;
  const float *w;
  float *y;
  int T, H, K, E, has_shared;
};

__global__ void __launch_bounds__(256) k_combine(CombineArgs a) {
  const int t = blockIdx.y;
  const int r = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (r >= a.H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < a.K; ++k) {
    const int e = a.ids[t * a.K + k];
    if (e < 0 || e >= a.E) continue;
    const float wk = a.w[t * a.K + k];
    const float4 v = *reinterpret_cast<const float4 *>(a.yd + ((size_t)t * (a.K + 1) + k) * a.H + r);
    s.x += wk * v.x;
    s.y += wk * v.y;
    s.z += wk * v.z;
    s.w += wk * v.w;
  }
  if (a.has_shared) {
    const float4 v = *reinterpret_cast<const float4 *>(a.yd + ((size_t)t * (a.K + 1) + a.K) * a.H + r);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<float4 *>(a.y + (size_t)t * a.H + r) = s;
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

template <typename F>
int allow_lds(F *f, size_t bytes) {
  return (int)hipFuncSetAttribute(reinterpret_cast<const void *>(f),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int BITS>
int launch_gemms(const GroupArgs &gu, const GroupArgs &dn, dim3 grid_gu, dim3 grid_dn,
                 hipStream_t st) {
  using GU = GL<BITS, false>;
  using DN = GL<BITS, true>;
  if (allow_lds(k_grouped<BITS, false>, GU::BYTES) || allow_lds(k_grouped<BITS, true>, DN::BYTES))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((k_grouped<BITS, false>), grid_gu, dim3(256), GU::BYTES, st, gu);
  hipLaunchKernelGGL((k_grouped<BITS, true>), grid_dn, dim3(256), DN::BYTES, st, dn);
  return 0;
}

}  // namespace

int grouped_max_buckets(const moe_dims &d, int T) {
  const int routed = d.n_experts < T * d.top_k ? d.n_experts : T * d.top_k;
  return routed + d.has_shared;
}

int launch_expert_forward_grouped(const moe_dims &d, const moe_layer &L, const uint16_t *x,
                                  int T, const int32_t *ids, const float *w, float *y, void *ws,
                                  void *stream) {
  const WsLayout W = ws_layout(d, T);
  const BlobLayout B = blob_layout(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  Ctrl *ctrl = reinterpret_cast<Ctrl *>(base + W.ctrl);
  int32_t *bk = reinterpret_cast<int32_t *>(base + W.bk);
  float *h = reinterpret_cast<float *>(base + W.h);
  float *yd = reinterpret_cast<float *>(base + W.yd);
  const int maxB = grouped_max_buckets(d, T);
  hipStream_t st = S(stream);

  BucketArgs ba;
  ba.ids = ids;
  ba.bk = bk;
  ba.ctrl = ctrl;
  ba.T = T;
  ba.K = d.top_k;
  ba.E = d.n_experts;
  ba.has_shared = d.has_shared;
  ba.maxB = maxB;
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, st, ba);

  const int nchunk_pairs = (T + kNC - 1) / kNC;  // a bucket holds at most T pairs
  GroupArgs gu;
  gu.x = x;
  gu.hin = nullptr;
  gu.experts = L.experts;
  gu.shared = L.shared;
  gu.stride = L.expert_stride;
  gu.bk = bk;
  gu.out = h;
  gu.R = d.inter;
  gu.C = d.hidden;
  gu.E = d.n_experts;
  gu.maxB = maxB;
  gu.K1 = d.top_k + 1;
  gu.off_q0 = (int64_t)B.off[MOE_SEC_GATE_Q];
  gu.off_q1 = (int64_t)B.off[MOE_SEC_UP_Q];
  gu.off_sb0 = (int64_t)B.off[MOE_SEC_GATE_SB];
  gu.off_sb1 = (int64_t)B.off[MOE_SEC_UP_SB];
  GroupArgs dn = gu;
  dn.x = nullptr;
  dn.hin = h;
  dn.out = yd;
  dn.R = d.hidden;
  dn.C = d.inter;
  dn.off_q0 = dn.off_q1 = (int64_t)B.off[MOE_SEC_DOWN_Q];
  dn.off_sb0 = dn.off_sb1 = (int64_t)B.off[MOE_SEC_DOWN_SB];
  const dim3 grid_gu((unsigned)(d.inter / kRT), (unsigned)maxB, (unsigned)nchunk_pairs);
  const dim3 grid_dn((unsigned)(d.hidden / kRT), (unsigned)maxB, (unsigned)nchunk_pairs);
  int rc = d.bits == 4 ? launch_gemms<4>(gu, dn, grid_gu, grid_dn, st)
                       : launch_gemms<2>(gu, dn, grid_gu, grid_dn, st);
  if (rc) return rc;

  CombineArgs ca;
  ca.yd = yd;
  ca.ids = ids;
  ca.w = w;
  ca.y = y;
  ca.T = T;
  ca.H = d.hidden;
  ca.K = d.top_k;
  ca.E = d.n_experts;
  ca.has_shared = d.has_shared;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((d.hidden / 4 + 255) / 256), (unsigned)T), dim3(256),
                     0, st, ca);
  return (int)hipGetLastError();
}

}  // namespace moe
