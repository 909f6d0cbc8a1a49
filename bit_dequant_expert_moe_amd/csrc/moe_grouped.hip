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
//   k_xprep      x of the batch in the B-operand layout, with group sums.
//   k_grouped    dequantising grouped GEMM on the matrix cores for one
//                (bucket, 64-row tile, 16-pair chunk):
//                  gate/up: h = silu(Gate x) * (Up x) for every pair, written
//                           as the B operand of the down pass;
//                  down:    yd = Down h for every pair.
//   k_combine    y[t] = sum_k w[t][k] yd[t][k] + yd[t][shared], in that order.
//
// Matrix-core arithmetic.  A group of 64 weights of a row shares (s, z), so
//   sum_c (s q_c + z) b_c = s * sum_c q_c b_c + z * sum_c b_c.
// The codes enter v_mfma_f32_16x16x32_bf16 as bf16 values 128 + q (exact: one
// v_and_or_b32 puts two 4-bit fields into the mantissas of a pair of bf16
// 128.0); the product with the bf16 activations is exact and the MFMA sums in
// fp32.  Per group the partial result P gives sum q b = P - 128 * sum b, so
// the group adds s P + (z - 128 s) sum b: the scale term in fp32 per group,
// the bias terms of a staged chunk's four groups as one fp32 16x16x4 MFMA.
// x is bf16 already; h (fp32) enters as bf16 hi + bf16 lo, two MFMAs, ~16
// significant bits.
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
constexpr int kNC = 16;         // pairs per block (one 16-wide MFMA tile; one work item)
constexpr int kKC = 256;        // columns per staged chunk
constexpr int kGC = kKC / kGroup;  // groups per chunk (4)
constexpr int kSl = kKC / 8;    // 8-column slices per chunk (32)
static_assert(kRT == kGroup, "a gate/up row tile is one group of the down columns");

// ---------------------------------------------------------------------------
// Buckets.  Layout of the int32 array bk (maxB = min(E, T K) + has_shared):
//   bk[0]                       number of buckets nb
//   bk[1 + j]                   expert of bucket j (E = the shared expert)
//   bk[1 + maxB + j], j <= nb   first pair of bucket j; bk[1 + maxB + nb] = total
//   bk[2 + 2 maxB + p]          pair code t (K + 1) + slot (slot K = shared),
//                               p < T (K + 1) = pair_cap
//   bk[2 + 2 maxB + pair_cap]   number of work items
//   bk[3 + 2 maxB + pair_cap + i]  work item i = bucket << 16 | chunk: the pairs
//                               kNC chunk .. kNC chunk + kNC - 1 of the bucket
//                               (bucket < maxB <= 1025 and chunk < T K / kNC
//                               <= 2048 even when a token repeats an expert)
// One GEMM block per (row tile, work item): no block is launched for an
// empty chunk of a bucket.
// ---------------------------------------------------------------------------

// Work item = bucket << kItemShift | chunk.
constexpr int kItemShift = 16;
static_assert((kMaxT * kMaxK + kNC - 1) / kNC < (1 << kItemShift), "chunk field holds every chunk");
static_assert((kMaxE + 1) < (1 << (31 - kItemShift)), "bucket field holds every bucket");

// Upper bound of the number of work items for T tokens.
__host__ __device__ constexpr int max_items(int E, int T, int K, int has_shared) {
  return (E < T * K ? E : T * K) + (T * K + kNC - 1) / kNC + (has_shared ? (T + kNC - 1) / kNC : 0);
}
// ---------------------------------------------------------------------------
struct BucketArgs {
  const int32_t *ids;
  int32_t *bk;
  Ctrl *ctrl;
  int T, K, E, has_shared, maxB, pair_cap;
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
  // work items: routed buckets in bucket order, then the shared bucket
  const int nz = (c + kNC - 1) / kNC;
  int nitems;
  const int ioff = block_exscan(nz, s_wtot, &nitems);
  int32_t *items = a.bk + 3 + 2 * a.maxB + a.pair_cap;
  for (int z = 0; z < nz; ++z) items[ioff + z] = (j << kItemShift) | z;
  if (tid == 0) {
    if (a.has_shared) {
      const int nzs = (a.T + kNC - 1) / kNC;
      for (int z = 0; z < nzs; ++z) items[nitems + z] = (nrb << kItemShift) | z;
      nitems += nzs;
    }
    a.bk[2 + 2 * a.maxB + a.pair_cap] = nitems;
  }
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
//
// B operands are read straight from global memory (L2-resident: x and h of the
// batch are a few MB) in the layout the matrix cores take, written by the
// producers: k_xprep for x, the gate/up epilogue for h.  Per 8-column slice s
// of a row of B: one 16-byte bf16x8 in the order (c0, c4, c1, c5, c2, c6, c3,
// c7) (x), or two (h as bf16 hi, then bf16 lo); per group of 64 columns the
// fp32 sum of the operand values (x, or hi + lo).  A block stages the codes,
// the scales and its 16 B columns of each chunk in LDS.
// ---------------------------------------------------------------------------
struct GroupArgs {
  const uint4 *bop;    // B operand: [rows of B][C / 8][BV] uint4
  const float *bsum;   // [rows of B][C / 64] group sums
  const uint8_t *experts, *shared;
  int64_t stride;
  const int32_t *bk;
  uint4 *hb;           // gate/up output: h as B operand of the down pass
  float *hs;           //   and its group sums
  float *yd;           // down output: [T (K+1)][H]
  int R, C;            // rows and columns of the matrices of this pass
  int E, maxB, K1;     // K1 = K + 1 (pair code = token K1 + slot)
  int pair_cap;        // T (K + 1): size of the pair-code list
  int64_t off_q0, off_q1, off_sb0, off_sb1;  // second matrix unused for down
  uint32_t bop_bytes, bsum_bytes;  // sizes of the bop and bsum areas (< kNoLoad)
};

template <int BITS, bool DOWN>
struct GL {  // LDS geometry
  static constexpr int NMAT = DOWN ? 1 : 2;
  static constexpr int RW = kKC * BITS / 32 + 2;  // words per staged row (+2 against bank conflicts)
  static constexpr int BV = DOWN ? 2 : 1;         // uint4 per (B row, slice)
  static constexpr int BCS = kSl * BV + 1;        // uint4 per staged B column (+1 against bank conflicts)
  static constexpr int BPT = kNC * kSl * BV / 256;  // B pieces per thread
  static constexpr int A_U32 = NMAT * kRT * RW;
  // gate/up: float2 (s, z - 128 s) per row and group; down: the (s, z) words
  // (the smaller area keeps three down blocks within a compute unit's LDS);
  // group-major ([matrix][group][row]), so that a lane's four output rows are
  // 16 or 32 contiguous bytes and the four row quads of a wave fall in
  // different banks
  static constexpr int SB_U32 = NMAT * kRT * kGC * (DOWN ? 1 : 2);
  static constexpr int B_U32 = kNC * BCS * 4;
  static constexpr int XS_U32 = kNC * kGC;
  static constexpr int BUF_U32 = A_U32 + SB_U32 + B_U32 + XS_U32;
  static constexpr size_t BYTES = 2 * (size_t)BUF_U32 * 4;
  static constexpr int PPR = kKC * BITS / 128;    // 16-byte pieces per staged row
  static constexpr int APT = NMAT * kRT * PPR / 256;  // A pieces per thread
  static_assert(APT >= 1 && (NMAT * kRT * PPR) % 256 == 0, "A pieces tile the block");
  static_assert(BPT >= 1 && (kNC * kSl * BV) % 256 == 0, "B pieces tile the block");
  static_assert((A_U32 + SB_U32) % 4 == 0, "B area 16-byte aligned");
};

// Two bf16 (hi half, lo half) of 128 + the fields selected by mask m, with
// M = 0x43004300 (the pair 128, 128).  Plain C, so that the hazard checks
// that keep a VALU write from overtaking an MFMA still reading the register
// see it; m and M arrive in registers (see Unpack), so the compiler can form
// one v_and_or_b32 (VOP3 takes no literal operand on this target).
__device__ __forceinline__ uint32_t magic_pair(uint32_t v, uint32_t m, uint32_t M) {
  return (v & m) | M;
}

// The unpack constants, held in registers: the field mask in an SGPR, the
// magic pair in a VGPR (an empty asm statement hides their values from
// constant folding, which would otherwise split each v_and_or_b32 into a
// v_and_b32 and a v_or_b32 with literals).
struct Unpack {
  uint32_t m, M;
  template <int BITS>
  __device__ static Unpack make() {
    Unpack u;
    u.m = BITS == 4 ? 0x000F000Fu : 0x00030003u;
    u.M = 0x43004300u;
    asm volatile("" : "+s"(u.m));
    asm volatile("" : "+v"(u.M));
    return u;
  }
};

// A operand of one 8-column slice: bf16 128 + q in the order
// (c0, c4, c1, c5, c2, c6, c3, c7).  For 2-bit codes the slice is one half
// (16 bits) of a word.
template <int BITS>
__device__ __forceinline__ bf16x8 a_slice(uint32_t word, int half, const Unpack &k) {
  uint32_t p[4];
  if (BITS == 4) {
    p[0] = magic_pair(word, k.m, k.M);
    p[1] = magic_pair(word >> 4, k.m, k.M);
    p[2] = magic_pair(word >> 8, k.m, k.M);
    p[3] = magic_pair(word >> 12, k.m, k.M);
  } else {
    const uint32_t h16 = half ? (word >> 16) : (word & 0xFFFFu);
    const uint32_t v = h16 | (h16 << 8);  // c_{j+4} lands 16 bits above c_j
    p[0] = magic_pair(v, k.m, k.M);
    p[1] = magic_pair(v >> 2, k.m, k.M);
    p[2] = magic_pair(v >> 4, k.m, k.M);
    p[3] = magic_pair(v >> 6, k.m, k.M);
  }
  uint4 u = make_uint4(p[0], p[1], p[2], p[3]);
  return __builtin_bit_cast(bf16x8, u);
}

// Loads through buffer resources: 32-bit unsigned byte offsets from a base
// held in scalar registers, range-checked against the resource's size.  An
// offset at or past the size returns zeros without a memory access, which is
// how a padding column or an idle thread issues its load: every load of the
// pipeline is issued on every path.
constexpr uint32_t kNoLoad = 0xFFFFFF00u;  // past every area (sizes are checked on the host)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t area_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// An empty volatile asm that reads and writes a loaded value: the wait for
// its load lands here, on every path, and not inside a conditional store that
// uses it (a wait inside a branch leaves the register pending on the other
// path, and the next load into it then waits for every load in flight).
__device__ __forceinline__ void settle(uint4 &u) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {u.x, u.y, u.z, u.w};
  __asm__ volatile("" : "+v"(v));
  u = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void settle(float &f) { __asm__ volatile("" : "+v"(f)); }

// (x0..x7 as pairs (x0,x1),(x2,x3),(x4,x5),(x6,x7)) -> (x0,x4),(x1,x5),(x2,x6),(x3,x7)
__device__ __forceinline__ uint4 b_order(uint4 q) {
  uint4 r;
  r.x = (q.x & 0xFFFFu) | (q.z << 16);
  r.y = (q.x >> 16) | (q.z & 0xFFFF0000u);
  r.z = (q.y & 0xFFFFu) | (q.w << 16);
  r.w = (q.y >> 16) | (q.w & 0xFFFF0000u);
  return r;
}

// x of the batch as B operand of the gate/up pass: one thread per slice.
struct XPrepArgs {
  const uint16_t *x;
  uint4 *xb;
  float *xs;
  int T, H;
};

__global__ void __launch_bounds__(256) k_xprep(XPrepArgs a) {
  const int ns = a.H / 8;
  const int i = blockIdx.x * 256 + threadIdx.x;  // slice over all tokens
  // (T H / 8 is a multiple of 8: whole groups are in or out of range)
  const bool in = i < a.T * ns;
  const uint4 v = in ? reinterpret_cast<const uint4 *>(a.x)[i] : make_uint4(0, 0, 0, 0);
  float part = bf16f(v.x & 0xFFFFu) + bf16f(v.x >> 16) + bf16f(v.y & 0xFFFFu) +
               bf16f(v.y >> 16) + bf16f(v.z & 0xFFFFu) + bf16f(v.z >> 16) +
               bf16f(v.w & 0xFFFFu) + bf16f(v.w >> 16);
  if (in) a.xb[i] = b_order(v);
  // a group is 8 consecutive slices: 8 consecutive lanes
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  part += __shfl_xor(part, 4, 64);
  if (in && (i & 7) == 0) a.xs[i >> 3] = part;
}

// Minimum waves per SIMD the register allocation must allow: three, so that
// three blocks of either pass fit a compute unit where LDS allows (the down
// pass's does; with its 53 KB a 170-register allocation would cost one block).
#ifndef MOE_GROUPED_MINW
#define MOE_GROUPED_MINW 3
#endif

// Row tiles per block of the down pass: its rows are short (C = I = 1024, four
// chunks), so one block runs the chunks of consecutive row tiles as one
// pipeline and the memory latency of a block's first chunks is paid once.
#ifndef MOE_GROUPED_DN_TILES
#define MOE_GROUPED_DN_TILES 2
#endif

template <int BITS, bool DOWN>
__global__ void __launch_bounds__(256, MOE_GROUPED_MINW) k_grouped(GroupArgs a) {
  using G = GL<BITS, DOWN>;
  constexpr int RTL = DOWN ? MOE_GROUPED_DN_TILES : 1;  // row tiles per block
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float s_hsum[4][16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, col = lane & 15;
  const int32_t *items = a.bk + 2 + 2 * a.maxB + a.pair_cap;
  if ((int)blockIdx.y >= items[0]) return;
  const int item = items[1 + blockIdx.y];
  const int j = item >> kItemShift;
  const int e = a.bk[1 + j];
  const int p0 = a.bk[1 + a.maxB + j], p1 = a.bk[2 + a.maxB + j];
  const int pbase = p0 + kNC * (item & ((1 << kItemShift) - 1));
  if (pbase >= p1) return;
  const int nn = min(kNC, p1 - pbase);
  const int32_t *pairs = a.bk + 2 + 2 * a.maxB + pbase;
  const uint8_t *blob = e == a.E ? a.shared : a.experts + (size_t)e * a.stride;
  const int row0 = kRT * RTL * (int)blockIdx.x;
  const size_t rbytes = (size_t)a.C * BITS / 8;
  const int groups = a.C / kGroup;
  const int nslices = a.C / 8;
  const int nchunks = a.C / kKC;
  // B columns of this block: the pair (down) or its token (gate/up) of each
  // of the kNC columns; padding columns are staged as zeros
  const int code = col < nn ? pairs[col] : 0;  // this lane's output column
  const bool bvalid = col < nn;

  // ---- per chunk: A pieces, scales, B columns and their sums to LDS ---------
  // Two register sets hold the next two chunks in flight while the current
  // one is computed from LDS (the pass is bound by bytes in flight).
  struct Regs {
    uint4 ra[G::APT];
    uint4 rsb;
    uint4 rb[G::BPT];
    float rxs;
  };
  // Byte offsets of this thread's loads at chunk 0, resolved once (a load
  // whose address depends on another load inside the pipeline would wait
  // for every load issued before it; loads complete in order).  Every load
  // of the pipeline is issued unconditionally, so that the wait before a
  // chunk is staged counts only the loads issued before it: a padding
  // column, or a thread with no scale word or group sum, loads at kNoLoad
  // and stages zeros.
  const __amdgpu_buffer_rsrc_t rs_blob = area_rsrc(blob, 0x7FFFFFFFu);
  const __amdgpu_buffer_rsrc_t rs_b = area_rsrc(a.bop, a.bop_bytes);
  const __amdgpu_buffer_rsrc_t rs_s = area_rsrc(a.bsum, a.bsum_bytes);
  uint32_t aoff[G::APT];
#pragma unroll
  for (int i = 0; i < G::APT; ++i) {
    const int pc = tid + 256 * i;
    const int mat = pc / (kRT * G::PPR), rr = (pc / G::PPR) % kRT, c16 = pc % G::PPR;
    aoff[i] = (uint32_t)((mat ? a.off_q1 : a.off_q0) + (int64_t)(row0 + rr) * (int64_t)rbytes) +
              c16 * 16;
  }
  uint32_t boff[G::BPT];
#pragma unroll
  for (int i = 0; i < G::BPT; ++i) {
    const int bc = (tid + 256 * i) / (kSl * G::BV), rest = (tid + 256 * i) % (kSl * G::BV);
    boff[i] = kNoLoad;
    if (bc < nn) {
      const int pcode = pairs[bc];
      const uint32_t brow = DOWN ? pcode : pcode / a.K1;
      boff[i] = (brow * (uint32_t)nslices * G::BV + rest) * 16u;
    }
  }
  uint32_t soff = kNoLoad;
  if (tid < kNC * kGC && tid / kGC < nn) {
    const int pcode = pairs[tid / kGC];
    const uint32_t brow = DOWN ? pcode : pcode / a.K1;
    soff = (brow * (uint32_t)groups + tid % kGC) * 4u;
  }
  const bool sbok = tid < G::NMAT * kRT;
  uint32_t sboff = kNoLoad;
  if (sbok) {
    const int mat = tid / kRT, rr = tid % kRT;
    sboff = (uint32_t)((mat ? a.off_sb1 : a.off_sb0) + (int64_t)(row0 + rr) * groups * 4);
  }
  // chunk c's offsets: the chunk-0 offset plus the chunk's, or kNoLoad
  auto at = [](uint32_t off0, uint32_t step) { return off0 == kNoLoad ? kNoLoad : off0 + step; };
  // virtual chunk vc: column chunk vc % nchunks of row tile vc / nchunks
  const int nv = RTL * nchunks;
  auto load_chunk = [&](int vc, Regs &R) {
    const int c = vc & (nchunks - 1), tile = vc / nchunks;
    const uint32_t arow = (uint32_t)(tile * kRT) * (uint32_t)rbytes;
#pragma unroll
    for (int i = 0; i < G::APT; ++i)
      R.ra[i] = bload16(rs_blob, aoff[i] + arow + c * (kKC * BITS / 8));
    R.rsb = bload16(rs_blob, at(sboff, (uint32_t)(tile * kRT * groups * 4) + c * kGC * 4));
#pragma unroll
    for (int i = 0; i < G::BPT; ++i) R.rb[i] = bload16(rs_b, at(boff[i], c * kSl * G::BV * 16));
    R.rxs = bload4f(rs_s, at(soff, c * kGC * 4));
  };
  auto store_chunk = [&](int buf, Regs &R) {
    settle(R.rsb);
#pragma unroll
    for (int i = 0; i < G::BPT; ++i) settle(R.rb[i]);
    settle(R.rxs);
    uint32_t *A = lds + (size_t)buf * G::BUF_U32;
    uint32_t *SB = A + G::A_U32;
    uint4 *Bq = reinterpret_cast<uint4 *>(SB + G::SB_U32);
    float *XS = reinterpret_cast<float *>(SB + G::SB_U32 + G::B_U32);
#pragma unroll
    for (int i = 0; i < G::APT; ++i) {
      const int pc = tid + 256 * i;
      const int mat = pc / (kRT * G::PPR), rr = (pc / G::PPR) % kRT, c16 = pc % G::PPR;
      uint32_t *dst = A + (mat * kRT + rr) * G::RW + c16 * 4;
      dst[0] = R.ra[i].x;
      dst[1] = R.ra[i].y;
      dst[2] = R.ra[i].z;
      dst[3] = R.ra[i].w;
    }
    const uint32_t w4[4] = {R.rsb.x, R.rsb.y, R.rsb.z, R.rsb.w};
    if (DOWN) {
      if (tid < kRT) {
#pragma unroll
        for (int g = 0; g < kGC; ++g) SB[g * kRT + tid] = w4[g];
      }
    } else if (sbok) {
      // per group (s, z - 128 s): the MFMA sums (128 + q) b, so
      // s sum q b + z sum b = s P + (z - 128 s) X
      const int mat = tid / kRT, rr = tid % kRT;
      float2 *dst = reinterpret_cast<float2 *>(SB);
#pragma unroll
      for (int g = 0; g < kGC; ++g) {
        const float sc = bf16f(w4[g] & 0xFFFFu), zb = bf16f(w4[g] >> 16);
        dst[(mat * kGC + g) * kRT + rr] = make_float2(sc, fmaf(-128.f, sc, zb));
      }
    }
#pragma unroll
    for (int i = 0; i < G::BPT; ++i) {
      const int pc = tid + 256 * i;
      const int bc = pc / (kSl * G::BV), rest = pc % (kSl * G::BV);
      Bq[bc * G::BCS + rest] = R.rb[i];
    }
    if (tid < kNC * kGC) XS[tid] = R.rxs;
  };

  f32x4 acc[G::NMAT];
#pragma unroll
  for (int m = 0; m < G::NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ar = wave * 16 + col;  // A row of this lane within the tile
  const Unpack uk = Unpack::make<BITS>();

  auto compute_chunk = [&](int buf) {
    const uint32_t *A = lds + (size_t)buf * G::BUF_U32;
    const uint32_t *SB = A + G::A_U32;
    const uint4 *Bq = reinterpret_cast<const uint4 *>(SB + G::SB_U32);
    const float *XS = reinterpret_cast<const float *>(SB + G::SB_U32 + G::B_U32);
#pragma unroll
    for (int gi = 0; gi < kGC; ++gi) {
      f32x4 P[G::NMAT];
#pragma unroll
      for (int m = 0; m < G::NMAT; ++m) P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sl = 8 * gi + 4 * h + q;  // slice of this lane
        bf16x8 bv[G::BV];
#pragma unroll
        for (int u = 0; u < G::BV; ++u)
          bv[u] = __builtin_bit_cast(bf16x8, Bq[col * G::BCS + sl * G::BV + u]);
#pragma unroll
        for (int m = 0; m < G::NMAT; ++m) {
          const uint32_t w = A[(m * kRT + ar) * G::RW + (BITS == 4 ? sl : (sl >> 1))];
          const bf16x8 av = a_slice<BITS>(w, sl & 1, uk);
#pragma unroll
          for (int u = 0; u < G::BV; ++u)
            P[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[u], P[m], 0, 0, 0);
        }
      }
      // element v of this lane: row 4 q + v of the wave's 16, B column col;
      // the scale term here, the bias term once per chunk below
#pragma unroll
      for (int m = 0; m < G::NMAT; ++m) {
        float sc[4];
        if (DOWN) {
          const uint4 sb = *reinterpret_cast<const uint4 *>(SB + gi * kRT + wave * 16 + 4 * q);
          sc[0] = bf16f(sb.x & 0xFFFFu);
          sc[1] = bf16f(sb.y & 0xFFFFu);
          sc[2] = bf16f(sb.z & 0xFFFFu);
          sc[3] = bf16f(sb.w & 0xFFFFu);
        } else {
          const float4 *sz = reinterpret_cast<const float4 *>(
              reinterpret_cast<const float2 *>(SB) + (m * kGC + gi) * kRT + wave * 16 + 4 * q);
          const float4 s01 = sz[0], s23 = sz[1];
          sc[0] = s01.x;
          sc[1] = s01.z;
          sc[2] = s23.x;
          sc[3] = s23.z;
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = fmaf(sc[v], P[m][v], acc[m][v]);
      }
    }
    // bias term of the chunk's kGC groups, sum_g (z - 128 s)[row][g] X[g][col],
    // as one fp32 16x16x4 product: lane l supplies row l % 16, group l / 16 of
    // the wave's rows and group l / 16, column l % 16 of the group sums
    static_assert(kGC == 4, "one 16x16x4 product per chunk");
    const float xg = XS[col * kGC + q];
#pragma unroll
    for (int m = 0; m < G::NMAT; ++m) {
      float zp;
      if (DOWN) {
        const uint32_t sb = SB[q * kRT + wave * 16 + col];
        zp = fmaf(-128.f, bf16f(sb & 0xFFFFu), bf16f(sb >> 16));
      } else {
        zp = reinterpret_cast<const float2 *>(SB)[(m * kGC + q) * kRT + wave * 16 + col].y;
      }
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(zp, xg, acc[m], 0, 0, 0);
    }
  };

  // ---- software pipeline over the (virtual) column chunks -------------------
  // chunk c is computed from LDS buffer c & 1 while chunks c + 1 and c + 2
  // are in flight in the register sets.  The steady-state loop issues its
  // loads unconditionally, and so does the prologue (a row of one chunk loads
  // chunk 0 twice): with a load skipped on some path, the wait before a chunk
  // is staged would have to count as if no later load were in flight, which
  // drains the pipeline to one chunk.
  // Down pass: a row tile's outputs are written after its last chunk.
  const int orow0 = row0 + wave * 16 + 4 * q;  // first of this lane's 4 rows (tile 0)
  auto finish = [&](int vc) {
    if (DOWN && ((vc + 1) & (nchunks - 1)) == 0) {
      const int tile = vc / nchunks;
      if (bvalid) {
        const float4 o = make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
        *reinterpret_cast<float4 *>(a.yd + (size_t)code * a.R + orow0 + tile * kRT) = o;
      }
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  Regs R0, R1;
  load_chunk(0, R0);
  load_chunk(nv > 1 ? 1 : 0, R1);
  store_chunk(0, R0);
  __syncthreads();
  int c = 0;
  for (; c + 3 < nv; c += 2) {
    load_chunk(c + 2, R0);
    compute_chunk(0);
    finish(c);
    store_chunk(1, R1);
    __syncthreads();
    load_chunk(c + 3, R1);
    compute_chunk(1);
    finish(c + 1);
    store_chunk(0, R0);
    __syncthreads();
  }
  // the last one to three chunks: c is in buffer 0, c + 1 in R1
  if (c + 2 < nv) load_chunk(c + 2, R0);
  compute_chunk(0);
  finish(c);
  if (c + 1 < nv) {
    store_chunk(1, R1);
    __syncthreads();
    compute_chunk(1);
    finish(c + 1);
    if (c + 2 < nv) {
      store_chunk(0, R0);
      __syncthreads();
      compute_chunk(0);
      finish(c + 2);
    }
  }

  // ---- epilogue (gate/up) ---------------------------------------------------
  const int orow = orow0;
  if (!DOWN) {
    // h for 4 rows; with the neighbour's 4 (lane + 16) they form the 8-row
    // slice that lanes with even q write as the B operand of the down pass
    float hv[4], hsum = 0.f;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float g = acc[0][v], u = acc[1][v];
      hv[v] = g / (1.f + expf(-g)) * u;
      hi[v] = f2bf(hv[v]);
      lo[v] = f2bf(hv[v] - bf16f(hi[v]));
      hsum += bf16f(hi[v]) + bf16f(lo[v]);
    }
    const uint32_t h01 = hi[0] | (hi[1] << 16), h23 = hi[2] | (hi[3] << 16);
    const uint32_t l01 = lo[0] | (lo[1] << 16), l23 = lo[2] | (lo[3] << 16);
    const uint32_t nh01 = __shfl_down(h01, 16, 64), nh23 = __shfl_down(h23, 16, 64);
    const uint32_t nl01 = __shfl_down(l01, 16, 64), nl23 = __shfl_down(l23, 16, 64);
    if (bvalid && (q & 1) == 0) {
      uint4 *dst = a.hb + ((size_t)code * (a.R / 8) + orow / 8) * 2;
      dst[0] = b_order(make_uint4(h01, h23, nh01, nh23));
      dst[1] = b_order(make_uint4(l01, l23, nl01, nl23));
    }
    // group sum of the tile's 64 rows (= one group of the down columns)
    hsum += __shfl_xor(hsum, 16, 64);
    hsum += __shfl_xor(hsum, 32, 64);
    if (q == 0) s_hsum[wave][col] = hsum;
    __syncthreads();
    if (tid < 16 && tid < nn) {
      const float t4 = s_hsum[0][tid] + s_hsum[1][tid] + s_hsum[2][tid] + s_hsum[3][tid];
      a.hs[(size_t)pairs[tid] * (a.R / kGroup) + blockIdx.x] = t4;
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

// Dequantisation hook of the grouped GEMM's A operand: s q + z per code, with
// q = (128 + q) - 128 from the bf16 slices a_slice forms, element i of a
// slice being column i / 2 (i even) or i / 2 + 4 (i odd) of its 8 columns.
template <int BITS>
__global__ void __launch_bounds__(256) k_dequant_slices(DequantArgs a) {
  constexpr int CPW = 32 / BITS;
  const Unpack uk = Unpack::make<BITS>();
  const int wpr = a.cols / CPW;
  const size_t n = (size_t)a.rows * wpr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const int c0 = (int)(i - r * wpr) * CPW;
    const uint32_t w = a.q[i];
    float q[CPW];
#pragma unroll
    for (int half = 0; half < CPW / 8; ++half) {
      const uint4 v = __builtin_bit_cast(uint4, a_slice<BITS>(w, half, uk));
      const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q[8 * half + k] = bf16f(e[k] & 0xFFFFu) - 128.f;
        q[8 * half + k + 4] = bf16f(e[k] >> 16) - 128.f;
      }
    }
    store_dequant_word<CPW>(a, r, c0, q);
  }
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

// Allows `bytes` of dynamic LDS for kernel f; the default cap (64 KB) needs
// no attribute call (a runtime call per launch that the common sizes skip).
template <typename F>
int allow_lds(F *f, size_t bytes) {
  if (bytes <= 64 * 1024) return 0;
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
  timing::mark(MOE_ST_GATEUP);
  hipLaunchKernelGGL((k_grouped<BITS, false>), grid_gu, dim3(256), GU::BYTES, st, gu);
  timing::mark(MOE_ST_DOWN);
  hipLaunchKernelGGL((k_grouped<BITS, true>), grid_dn, dim3(256), DN::BYTES, st, dn);
  return 0;
}

}  // namespace

int launch_dequant_slices(const DequantArgs &a, int blocks, void *stream) {
  if (a.bits == 4)
    hipLaunchKernelGGL(k_dequant_slices<4>, dim3(blocks), dim3(256), 0, S(stream), a);
  else
    hipLaunchKernelGGL(k_dequant_slices<2>, dim3(blocks), dim3(256), 0, S(stream), a);
  return (int)hipGetLastError();
}

int grouped_max_buckets(const moe_dims &d, int T) {
  const int routed = d.n_experts < T * d.top_k ? d.n_experts : T * d.top_k;
  return routed + d.has_shared;
}

int grouped_bucket_words(const moe_dims &d, int T) {
  return 3 + 2 * grouped_max_buckets(d, T) + T * (d.top_k + 1) +
         max_items(d.n_experts, T, d.top_k, d.has_shared);
}

int launch_expert_forward_grouped(const moe_dims &d, const moe_layer &L, const uint16_t *x,
                                  int T, const int32_t *ids, const float *w, float *y, void *ws,
                                  void *stream) {
  const WsLayout W = ws_layout(d, T);
  const BlobLayout B = blob_layout(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  Ctrl *ctrl = reinterpret_cast<Ctrl *>(base + W.ctrl);
  int32_t *bk = reinterpret_cast<int32_t *>(base + W.bk);
  uint4 *xb = reinterpret_cast<uint4 *>(base + W.xb);
  float *xs = reinterpret_cast<float *>(base + W.xs);
  uint4 *hb = reinterpret_cast<uint4 *>(base + W.hb);
  float *hs = reinterpret_cast<float *>(base + W.hs);
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
  ba.pair_cap = T * (d.top_k + 1);
  timing::mark(MOE_ST_BUCKET);
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, st, ba);

  XPrepArgs xa;
  xa.x = x;
  xa.xb = xb;
  xa.xs = xs;
  xa.T = T;
  xa.H = d.hidden;
  hipLaunchKernelGGL(k_xprep, dim3((unsigned)(((size_t)T * d.hidden / 8 + 255) / 256)), dim3(256),
                     0, st, xa);

  const int nitems = max_items(d.n_experts, T, d.top_k, d.has_shared);
  GroupArgs gu;
  gu.bop = xb;
  gu.bsum = xs;
  gu.experts = L.experts;
  gu.shared = L.shared;
  gu.stride = L.expert_stride;
  gu.bk = bk;
  gu.hb = hb;
  gu.hs = hs;
  gu.yd = nullptr;
  gu.R = d.inter;
  gu.C = d.hidden;
  gu.E = d.n_experts;
  gu.maxB = maxB;
  gu.K1 = d.top_k + 1;
  gu.pair_cap = T * (d.top_k + 1);
  gu.off_q0 = (int64_t)B.off[MOE_SEC_GATE_Q];
  gu.off_q1 = (int64_t)B.off[MOE_SEC_UP_Q];
  gu.off_sb0 = (int64_t)B.off[MOE_SEC_GATE_SB];
  gu.off_sb1 = (int64_t)B.off[MOE_SEC_UP_SB];
  const size_t P = (size_t)T * (d.top_k + 1);
  const size_t area[4] = {(size_t)T * d.hidden * 2, (size_t)T * (d.hidden / kGroup) * 4,
                          P * d.inter * 4, P * (d.inter / kGroup) * 4};
  for (size_t v : area)
    if (v >= kNoLoad) return (int)hipErrorInvalidValue;  // beyond 32-bit buffer offsets
  gu.bop_bytes = (uint32_t)area[0];
  gu.bsum_bytes = (uint32_t)area[1];
  GroupArgs dn = gu;
  dn.bop = hb;
  dn.bsum = hs;
  dn.bop_bytes = (uint32_t)area[2];
  dn.bsum_bytes = (uint32_t)area[3];
  dn.hb = nullptr;
  dn.hs = nullptr;
  dn.yd = yd;
  dn.R = d.hidden;
  dn.C = d.inter;
  dn.off_q0 = dn.off_q1 = (int64_t)B.off[MOE_SEC_DOWN_Q];
  dn.off_sb0 = dn.off_sb1 = (int64_t)B.off[MOE_SEC_DOWN_SB];
  const dim3 grid_gu((unsigned)(d.inter / kRT), (unsigned)nitems);
  const dim3 grid_dn((unsigned)(d.hidden / (kRT * MOE_GROUPED_DN_TILES)), (unsigned)nitems);
  int rc = d.bits == 4 ? launch_gemms<4>(gu, dn, grid_gu, grid_dn, st)
                       : launch_gemms<2>(gu, dn, grid_gu, grid_dn, st);
  if (rc) return rc;

  timing::mark(MOE_ST_COMBINE);
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
