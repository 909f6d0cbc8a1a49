// moe_fused.hip -- the whole MoE layer for one token in one launch.
//
// Method: "Flash-MoE: Running a 397B Parameter Model on a Laptop"
// (hysenlabs.com), section "How the SSD expert streaming pipeline works":
// router -> softmax + top-K -> expert forward of the K selected experts and
// the shared expert -> combine.  "Flash-MoE: Running a 400 Billion Parameter
// Model on a MacBook" (mattcullerton.com), section "The Architecture": 4-bit
// experts dequantised inside the FMA inner loop.
//
// Why one launch: a decode layer moves ~40 MB, about 6 us of HBM time on
// MI355X, while a dependent kernel boundary costs ~1.7 us and a device-wide
// barrier across 256 workgroups ~2.3 us.  This kernel keeps every workgroup
// resident (one per CU) and replaces the two data dependencies of the layer
// with one-way exchanges:
//   * routing: each workgroup writes its logits as 64-bit words (fp32 bits,
//     epoch of the call); every workgroup reads the E words until all carry
//     the current epoch -- the data arrives with the signal -- and selects
//     the top-K itself (the selection is deterministic, so all agree);
//   * activations h: each gate/up wave writes its row of every slot as a
//     tagged 64-bit word as soon as it is computed.  The down rows of the
//     shared expert are split over all workgroups (16 each), those of routed
//     slot k over workgroups 64k .. 64k+63 (64 rows each), so a workgroup
//     reads the I words of two slots only (shared, own routed slot) until
//     all are current, into LDS for its down waves;
//   * routed down sums: the workgroup that computed routed rows r of slot k
//     writes their weighted sums as tagged words; the workgroup that owns
//     output rows r (16 per workgroup, those of its shared rows) reads the
//     four slots' sums of its rows (one reader per word) and forms
//     y = shared + slot 0 + .. + slot K-1 in that order.
// Every word that all workgroups read is written once per reader group
// (blockIdx % 8, one per XCD), so a cache line has at most 32 coherent
// readers: a line read coherently by all 256 CUs at once serialises at its
// memory channel for several microseconds.  Exchanged words travel through
// agent-scope relaxed atomics (coherent sc1 loads and stores); no cache
// writeback or invalidate is issued (issued by every CU at once, those cost
// tens of microseconds).
//
// Each workgroup has 8 waves (two per SIMD, so 256 VGPRs each): waves 0-3
// compute gate/up rows (one row of every slot each), waves 4-7 compute down
// rows (four shared rows and 16 rows of the own routed slot each).  Wave 4
// also selects the top-K and runs the reads of the exchanges.  Compared with
// every workgroup reading all five slots (one ~1 us round trip per slot at
// the end of the layer), this layout reads two slots and one small block of
// sums; with the publishing below, 1.2 us per layer less.
//
// Weight bytes are requested as soon as their addresses are known: router and
// x at launch, the shared expert once the router products are formed (issued
// at launch, its 7 MB delayed the router's 4 MB by ~0.5 us per layer), routed
// experts right after the top-K, gate/up rows first (the activation exchange
// waits on them; the down rows are needed only after it, ~1 us per layer
// faster than the reverse order).  Waits between waves of a workgroup read
// LDS only (a global or flat load in a spin loop would wait for every weight
// load the wave has in flight).
//
// Measured on MI355X (256 workgroups): one-way visibility of a coherent store
// to a polling workgroup is ~0.7 us; an all-gather round over 256 workgroups
// ~2.3-2.6 us, longer with more bytes polled per round and under HBM
// streaming.  Polling several slots per round, spreading the polls over more
// waves or more copies, and polling from the gate/up waves all measured
// slower than this layout.  Publishing from the gate/up waves directly, not
// through the polling wave, is ~0.5 us per layer faster: a wave waiting on a
// poll cannot publish.
//
// Residual mode (RES): the layer also runs the two steps around it on the
// residual stream r (fp32, updated in place): x = bf16(r / rms(r)) before the
// router, r += y after the combine.  Every workgroup normalises the whole
// vector itself (16 KB from L2; no extra exchange), and writes its own rows of
// r only after it has received the routed sums of those rows, which were
// formed from activations that every workgroup publishes only after it has
// read all of r: reads of r in any workgroup precede writes of r in every
// workgroup.
//
// Termination: every wait is bounded; a wait that times out sets bit 1 of
// the sticky error word and the kernel runs to completion.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_fused_dev.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace dev;

struct FusedArgs {
  const uint16_t *x, *router;
  const uint8_t *experts, *shared;
  int64_t stride;
  const int32_t *ids_in;  // given routing (then the router is skipped), or null
  const float *w_in;
  int32_t *ids_out;       // optional outputs
  float *w_out;
  float *y;
  Ctrl *ctrl;
  FCtrl *fc;
  uint64_t *tags;         // [kGroups][kMaxE] tagged logits
  uint64_t *htag;         // [kGroups][K+1][I] tagged activations
  uint64_t *ptag;         // [K][H] tagged routed down sums
  float *resid;           // residual mode: r, fp32 [H], read and updated in place
  uint16_t *x_out;        // residual mode: the normalised x, bf16 [H], or null
  int E, has_shared;
  int64_t off_gq, off_uq, off_dq, off_gsb, off_usb, off_dsb;
};

template <int BITS, int H, int I, int K, int RR, bool RES>
__global__ void __launch_bounds__(kNT, 1) k_layer1(FusedArgs a) {
  using Gm = Geo<BITS, H, I, K>;
  constexpr int COLS = Gm::COLS, PAIRS = Gm::PAIRS, LSEG = Gm::LSEG;
  constexpr int NSL = K + 1;  // slot K is the shared expert
  static_assert(NSL == kFusedSlots && I == kFusedI, "tagged activations are sized for these");
  __shared__ float s_red[kNT / 64][RR];
  __shared__ uint32_t s_xp[Gm::SEG_X][PAIRS];  // packed x pairs per segment
  __shared__ float2 s_cx[Gm::SEG_X];           // (1024 * sum of pairs, sum of x)
  __shared__ float s_hb[2][I];                 // h of the shared and the own routed slot
  __shared__ int32_t s_ids[K];
  __shared__ float s_w[K];
  __shared__ uint32_t s_cnt[NSL];              // gate/up rows published, per slot
  __shared__ uint32_t s_hready[2];             // s_hb[i] filled
  __shared__ float s_part[K][Gm::D_ROWS];      // routed sums of this workgroup's y rows
  __shared__ uint32_t s_pready;                // s_part filled
  __shared__ uint32_t s_epoch;
  __shared__ uint32_t s_ready;                 // routing selected
  __shared__ uint32_t s_dissued;               // gate/up waves that issued their routed loads
  __shared__ float s_ss[kNT / 64];             // residual mode: sum of r^2 per wave
  __shared__ uint4 s_xn[RES ? H / 8 : 1];      // residual mode: normalised x, bf16

  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = b % kGroups;
  const bool routing = a.ids_in == nullptr;
  constexpr int rr = RR;  // router rows per workgroup (E <= RR * kG)

  // the epoch of this call (calls completed + 1) is read first by the last
  // wave, which needs nothing before barrier (A), and published there
  constexpr int kEpochTid = kNT - 64;
  // (the other threads' value is never used; a non-constant one keeps the
  // compiler from folding the +1 into the branch, which would wait for the
  // load right there)
  uint32_t epoch_done = (uint32_t)a.E;
  if (tid == kEpochTid) epoch_done = ld_rlx(&a.fc->epoch[grp][0]);
  if (tid < NSL) s_cnt[tid] = 0u;
  if (tid < 2) s_hready[tid] = 0u;
  if (tid == 0) {
    s_ready = 0u;
    s_dissued = 0u;
    s_pready = 0u;
  }

  // ---- router loads (all threads) -------------------------------------------
  // thread tid owns x chunk tid + kNT j (8 columns); in residual mode it loads
  // the fp32 r of those columns instead and x is formed by norm_x below
  uint4 rw[RR * Gm::RXC], rx[Gm::RXC];
  float4 rf[RES ? 2 * Gm::RXC : 1];
  if (RES) {
#pragma unroll
    for (int j = 0; j < Gm::RXC; ++j) {
      const float4 *p = reinterpret_cast<const float4 *>(a.resid + (size_t)(tid + kNT * j) * 8);
      rf[2 * j] = p[0];
      rf[2 * j + 1] = p[1];
    }
  }
  if (routing) {
    if (!RES) {
#pragma unroll
      for (int j = 0; j < Gm::RXC; ++j)
        rx[j] = *reinterpret_cast<const uint4 *>(a.x + (size_t)(tid + kNT * j) * 8);
    }
#pragma unroll
    for (int i = 0; i < RR * Gm::RXC; ++i) {
      const int row = i / Gm::RXC, e = b * rr + row;
      const int ch = tid + kNT * (i % Gm::RXC);
      // rows past E read row E-1 and are never published (loads stay
      // unconditional so the load counter can be tracked statically)
      const int ec = e < a.E ? e : a.E - 1;
      rw[i] = *reinterpret_cast<const uint4 *>(a.router + (size_t)ec * H + (size_t)ch * 8);
    }
  }
  // Residual mode, all waves, once: x = bf16(r / sqrt(mean(r^2) + eps)) into
  // rx and s_xn.  The per-wave sums are added in wave order, so every thread
  // of every workgroup uses the same scale.  The two barriers order LDS only.
  auto norm_x = [&]() {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2 * Gm::RXC; ++j) {
      ss = fmaf(rf[j].x, rf[j].x, ss);
      ss = fmaf(rf[j].y, rf[j].y, ss);
      ss = fmaf(rf[j].z, rf[j].z, ss);
      ss = fmaf(rf[j].w, rf[j].w, ss);
    }
    ss = wave_sum64(ss);
    if (lane == 0) s_ss[wave] = ss;
    lds_release();
    __builtin_amdgcn_s_barrier();
    lds_acquire();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNT / 64; ++w) tot += s_ss[w];
    const float inv = 1.f / sqrtf(tot * (1.f / (float)H) + kRmsEps);
#pragma unroll
    for (int j = 0; j < Gm::RXC; ++j) {
      const float4 lo = rf[2 * j], hi = rf[2 * j + 1];
      rx[j] = make_uint4(f2bf(lo.x * inv) | (f2bf(lo.y * inv) << 16),
                         f2bf(lo.z * inv) | (f2bf(lo.w * inv) << 16),
                         f2bf(hi.x * inv) | (f2bf(hi.y * inv) << 16),
                         f2bf(hi.z * inv) | (f2bf(hi.w * inv) << 16));
      s_xn[tid + kNT * j] = rx[j];
      if (b == 0 && a.x_out)
        *reinterpret_cast<uint4 *>(a.x_out + (size_t)(tid + kNT * j) * 8) = rx[j];
    }
    lds_release();
    __builtin_amdgcn_s_barrier();
    lds_acquire();
  };
  auto router_partials = [&]() {
    float part[RR];
#pragma unroll
    for (int row = 0; row < RR; ++row) part[row] = 0.f;
#pragma unroll
    for (int i = 0; i < RR * Gm::RXC; ++i) {
      const uint4 wv = rw[i], xv = rx[i % Gm::RXC];
      float acc = part[i / Gm::RXC];
      acc = dot2b(wv.x, xv.x, acc);
      acc = dot2b(wv.y, xv.y, acc);
      acc = dot2b(wv.z, xv.z, acc);
      acc = dot2b(wv.w, xv.w, acc);
      part[i / Gm::RXC] = acc;
    }
#pragma unroll
    for (int row = 0; row < RR; ++row) {
      const float v = wave_sum64(part[row]);
      if (lane == 0) s_red[wave][row] = v;
    }
  };

  if (wave < kGuWaves) {
    // ========================= gate/up waves ================================
    const int r = b * Gm::GU_ROWS + wave;  // this wave's row of every slot
    const size_t rbytes = (size_t)H * BITS / 8;
    const int groups = H / kGroup;
    // x segments to stage (one per thread of the gate/up waves)
    const int xs = tid;
    uint4 xr[Gm::XLD];
    if (!RES) {
#pragma unroll
      for (int t = 0; t < Gm::XLD; ++t)
        xr[t] = *reinterpret_cast<const uint4 *>(a.x + (size_t)(xs % Gm::SEG_X) * COLS + 8 * t);
    }
    uint4 gq[NSL][LSEG], uq[NSL][LSEG];
    uint32_t gsb[NSL][LSEG], usb[NSL][LSEG];
    // byte offsets inside a blob, the same for every expert
    uint32_t o_gq[LSEG], o_uq[LSEG], o_gsb[LSEG], o_usb[LSEG];
#pragma unroll
    for (int j = 0; j < LSEG; ++j) {
      const int sg = lane + 64 * j;
      o_gq[j] = (uint32_t)(a.off_gq + (int64_t)r * rbytes + sg * 16);
      o_uq[j] = (uint32_t)(a.off_uq + (int64_t)r * rbytes + sg * 16);
      o_gsb[j] = (uint32_t)(a.off_gsb + ((int64_t)r * groups + sg * COLS / kGroup) * 4);
      o_usb[j] = (uint32_t)(a.off_usb + ((int64_t)r * groups + sg * COLS / kGroup) * 4);
    }
    auto load_rows = [&](int slot, const uint8_t *bl) {
      const __amdgpu_buffer_rsrc_t rs = blob_rsrc(bl);
#pragma unroll
      for (int j = 0; j < LSEG; ++j) {
        gq[slot][j] = bld16(rs, o_gq[j]);
        uq[slot][j] = bld16(rs, o_uq[j]);
        gsb[slot][j] = bld4(rs, o_gsb[j]);
        usb[slot][j] = bld4(rs, o_usb[j]);
      }
      // keep the slots' loads in issue order = consumption order (the load
      // counter completes in order)
      __builtin_amdgcn_sched_barrier(0);
    };
    if (RES) {
      norm_x();
#pragma unroll
      for (int t = 0; t < Gm::XLD; ++t) xr[t] = s_xn[(xs % Gm::SEG_X) * (COLS / 8) + t];
    }
    if (routing) router_partials();
    // without a shared expert slot K reads expert 0 and is never used
    load_rows(K, a.has_shared ? a.shared : a.experts);
    // x pairs and per-segment corrections, one code word at a time, to LDS
    if (xs < Gm::SEG_X) {
      float C = 0.f, X = 0.f;
      const uint32_t *xw = reinterpret_cast<const uint32_t *>(&xr[0]);
      const int xkey = xp_key<PAIRS>(xs);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        constexpr int CPW = 32 / BITS;  // columns per code word
        float v[CPW];
#pragma unroll
        for (int m = 0; m < CPW / 2; ++m) {
          const uint32_t pr = xw[wd * CPW / 2 + m];
          v[2 * m] = bf16f(pr & 0xFFFFu);
          v[2 * m + 1] = bf16f(pr >> 16);
        }
#pragma unroll
        for (int c = 0; c < CPW; ++c) X += v[c];
        if (BITS == 4) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float sc = (p & 1) ? 0.0625f : 1.f;
            const uint32_t pr = pack_h2(v[p] * sc, v[p + 4] * sc);
            s_xp[xs][(4 * wd + p) ^ xkey] = pr;
            C += h2_sum(pr);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int e = k < 5 ? k : k - 5;
            const float sc = 1.f / (float)(1 << (2 * e));
            const uint32_t pr = pack_h2(v[k] * sc, v[k + 8] * sc);
            s_xp[xs][(8 * wd + k) ^ xkey] = pr;
            C += h2_sum(pr);
          }
        }
      }
      s_cx[xs] = make_float2(1024.f * C, X);
    }
    auto gateup = [&](int slot) -> float {
      float pg = 0.f, pu = 0.f;
#pragma unroll
      for (int j = 0; j < LSEG; ++j) {
        const int sg = lane + 64 * j;
        const int xk = xp_key<PAIRS>(sg);
        uint32_t xp[PAIRS];
#pragma unroll
        for (int p = 0; p < PAIRS; p += 4) {
          const uint4 q = *reinterpret_cast<const uint4 *>(&s_xp[sg][p ^ xk]);
          xp[p] = q.x;
          xp[p + 1] = q.y;
          xp[p + 2] = q.z;
          xp[p + 3] = q.w;
        }
        const float2 cx = s_cx[sg];
        const float ag = seg_dot_x<BITS>(gq[slot][j], xp) - cx.x;
        const float au = seg_dot_x<BITS>(uq[slot][j], xp) - cx.x;
        pg += bf16f(gsb[slot][j] & 0xFFFFu) * ag + bf16f(gsb[slot][j] >> 16) * cx.y;
        pu += bf16f(usb[slot][j] & 0xFFFFu) * au + bf16f(usb[slot][j] >> 16) * cx.y;
      }
      pg = wave_sum64(pg);
      pu = wave_sum64(pu);
      return pg / (1.f + expf(-pg)) * pu;
    };
    __syncthreads();  // (A) router partials in s_red, x pairs in s_xp, epoch in s_epoch
    const uint32_t epoch = s_epoch;
    // publish h of (slot, this wave's row): one tagged copy per reader group,
    // then count the row for the exchange wave
    auto publish = [&](int slot, float hv) {
      if (lane < kGroups)
        __hip_atomic_store(&a.htag[((size_t)lane * NSL + slot) * I + b * Gm::GU_ROWS + wave],
                           ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(hv), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_fetch_add(&s_cnt[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    if (a.has_shared) publish(K, gateup(K));
    wait_lds(&s_ready, 1u);
    int eid[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      eid[k] = __builtin_amdgcn_readfirstlane(s_ids[k]);
      const bool ok = eid[k] >= 0 && eid[k] < a.E;
      // an invalid id reads expert 0 and contributes 0
      load_rows(k, a.experts + (size_t)(ok ? eid[k] : 0) * a.stride);
    }
    if (lane == 0)
      __hip_atomic_fetch_add(&s_dissued, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const bool ok = eid[k] >= 0 && eid[k] < a.E;
      publish(k, ok ? gateup(k) : 0.f);
    }
  } else {
    // =========================== down waves =================================
    // Output rows: the workgroup owns y rows b D_ROWS .. + D_ROWS; it computes
    // the shared expert's down rows there and adds the routed slots' sums,
    // which come from the workgroups that own those rows of each routed slot:
    // workgroup b computes the down rows O_ROWS (b % OWN_WG) .. + O_ROWS of
    // routed slot b / OWN_WG only, so it needs the activations of the shared
    // slot and of that one slot.
    const int dw = wave - kGuWaves;
    const bool xchg = dw == 0;  // this wave runs routing and the exchanges
    const int seg = lane % Gm::LPR;
    const size_t rbytes = (size_t)I * BITS / 8;
    const int groups = I / kGroup;
    const int ks = b / Gm::OWN_WG;  // the routed slot whose rows this workgroup computes
    const int obase = (b % Gm::OWN_WG) * Gm::O_ROWS + dw * Gm::O_ROWS_W;  // first row of this wave
    int rows[Gm::DLD];
#pragma unroll
    for (int ld = 0; ld < Gm::DLD; ++ld)
      rows[ld] = b * Gm::D_ROWS + dw * Gm::D_ROWS_W + ld * Gm::RPL + lane / Gm::LPR;
    // residual mode: r of this lane's output rows, read before any workgroup
    // can write r
    float rres[RES ? Gm::DLD : 1];
    if (RES) {
#pragma unroll
      for (int ld = 0; ld < Gm::DLD; ++ld) rres[ld] = a.resid[rows[ld]];
    }
    auto o_dq = [&](int row) -> uint32_t {
      return (uint32_t)(a.off_dq + (int64_t)row * rbytes + seg * Gm::DWORDS * 4);
    };
    auto o_dsb = [&](int row) -> uint32_t {
      return (uint32_t)(a.off_dsb + ((int64_t)row * groups + seg * Gm::DCOLS / kGroup) * 4);
    };
    auto ld_codes = [&](__amdgpu_buffer_rsrc_t rs, int row) -> uint4 {
      if (Gm::DWORDS == 4) return bld16(rs, o_dq(row));
      const uint2 v = bld8(rs, o_dq(row));
      return make_uint4(v.x, v.y, 0u, 0u);
    };
    // shared expert rows (issued once the router products are formed) and the
    // own routed slot's rows
    uint4 dqs[Gm::DLD], dqr[Gm::RDLD];
    uint32_t dsbs[Gm::DLD], dsbr[Gm::RDLD];
    if (RES) norm_x();
    if (routing) router_partials();
    {
      const __amdgpu_buffer_rsrc_t rs = blob_rsrc(a.has_shared ? a.shared : a.experts);
#pragma unroll
      for (int ld = 0; ld < Gm::DLD; ++ld) {
        dqs[ld] = ld_codes(rs, rows[ld]);
        dsbs[ld] = bld4(rs, o_dsb(rows[ld]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tid == kEpochTid) s_epoch = epoch_done + 1u;
    __syncthreads();  // (A)
    const uint32_t epoch = s_epoch;

    // ---- the exchanges (wave 4 only) ----
    // read this group's copy of `slot`; if every entry carries the current
    // epoch, move the values to s_hb[dst] for the down waves and return true
    auto try_consume = [&](int slot, int dst) -> bool {
      constexpr int NLD = I / 128;  // 16-byte loads per lane (two entries each)
      uint4 t[NLD];
      const uint32_t base = (uint32_t)(((size_t)grp * NSL + slot) * I * 8);
#pragma unroll
      for (int i = 0; i < NLD; ++i) t[i] = ld_coh16(a.htag, base + (uint32_t)(128 * i + 2 * lane) * 8u);
      bool ok = true;
#pragma unroll
      for (int i = 0; i < NLD; ++i) ok &= t[i].y == epoch && t[i].w == epoch;
      if (!__all(ok)) return false;
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        *reinterpret_cast<float2 *>(&s_hb[dst][hb_pos(128 * i + 2 * lane)]) =
            make_float2(__uint_as_float(t[i].x), __uint_as_float(t[i].z));
      lds_release();
      if (lane == 0) *lds(&s_hready[dst]) = 1u;
      return true;
    };
    // routed slots this workgroup has published (its four gate/up rows)
    int published = 0;
    auto count_published = [&]() {
      while (published < K && *lds(&s_cnt[published]) >= (uint32_t)kGuWaves) ++published;
    };
    long xspins = 0;  // one poll budget for the rest of the call
    auto timed_out = [&]() -> bool {
      if (++xspins <= kSpinMax) return false;
      if (lane == 0) atomicOr(&a.ctrl->err, 2u);
      return true;
    };
    // poll `slot` into s_hb[dst] until it is complete everywhere (a routed
    // slot only after this workgroup published it)
    auto exchange_until = [&](int slot, int dst) {
      while (true) {
        count_published();
        if ((slot == K || slot < published) && try_consume(slot, dst)) return;
        if (timed_out()) {
          if (lane == 0) *lds(&s_hready[dst]) = 1u;
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    // the routed sums of this workgroup's output rows: lane 16 k + i reads
    // slot k, row b D_ROWS + i (one reader per word)
    auto try_parts = [&]() -> bool {
      const int k = lane / Gm::D_ROWS, i = lane % Gm::D_ROWS;
      const uint2 t = ld_coh8(a.ptag, (uint32_t)(((size_t)k * H + b * Gm::D_ROWS + i) * 8));
      if (!__all(t.y == epoch)) return false;
      s_part[k][i] = __uint_as_float(t.x);
      lds_release();
      if (lane == 0) *lds(&s_pready) = 1u;
      return true;
    };

    if (xchg) {
      // 1. this workgroup's logits, one copy per reader group
      if (routing && lane < kGroups * rr) {
        const int rep = lane / rr, row = lane % rr, e = b * rr + row;
        if (e < a.E) {
          float l = 0.f;
#pragma unroll
          for (int w = 0; w < kNT / 64; ++w) l += s_red[w][row];
          const uint64_t v = ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(l);
          __hip_atomic_store(&a.tags[(size_t)rep * kMaxE + e], v, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // 2. routing: wait for every workgroup's tagged logits in this group's
      //    copy, select the top-K.  Lane l holds experts 128 i + 2 l + {0, 1}.
      if (routing) {
        // entries E .. 256 RR - 1 of the copy (within its kMaxE words) are
        // read but ignored, so every load is unconditional
        const uint64_t *tags_mine = a.tags + (size_t)grp * kMaxE;
        constexpr int NV = 4 * RR;
        static_assert(256 * RR <= kMaxE, "tag copy holds 256 RR entries");
        float v[NV];
        long spins = 0;
        // the first poll waits ~0.5 us: one issued before the last
        // workgroups' logits can be visible returns incomplete and costs a
        // whole round trip (~1.5 us under the shared-expert stream); waits
        // of 0.3 and 0.75 us measured between none and this one
        __builtin_amdgcn_s_sleep(19);
        while (true) {
          uint4 t[NV / 2];
#pragma unroll
          for (int i = 0; i < NV / 2; ++i) t[i] = ld_coh16(tags_mine, (uint32_t)(128 * i + 2 * lane) * 8u);
          bool ok = true;
#pragma unroll
          for (int i = 0; i < NV / 2; ++i) {
            const int idx = 128 * i + 2 * lane;
            ok &= (idx >= a.E || t[i].y == epoch) && (idx + 1 >= a.E || t[i].w == epoch);
            v[2 * i] = idx < a.E ? __uint_as_float(t[i].x) : __builtin_nanf("");
            v[2 * i + 1] = idx + 1 < a.E ? __uint_as_float(t[i].z) : __builtin_nanf("");
          }
          if (__all(ok)) break;
          if (++spins > kSpinMax) {
            if (lane == 0) atomicOr(&a.ctrl->err, 2u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        float sel_v[K];
        int sel_i[K];
        topk_select<K, NV>(v, lane, sel_v, sel_i);
        int id;
        float wk;
        topk_weights<K>(sel_v, sel_i, lane, id, wk);
        if (lane < K) {
          s_ids[lane] = id;
          s_w[lane] = wk;
          if (b == 0 && a.ids_out) a.ids_out[lane] = id;
          if (b == 0 && a.w_out) a.w_out[lane] = wk;
        }
      } else if (lane < K) {
        const int e = a.ids_in[lane];
        s_ids[lane] = e;
        s_w[lane] = a.w_in[lane];
        if ((e < 0 || e >= a.E) && b == 0) atomicOr(&a.ctrl->err, 1u);
      }
      lds_release();
      if (lane == 0) *lds(&s_ready) = 1u;
    } else {
      wait_lds(&s_ready, 1u);
    }

    // own routed rows: issued after the gate/up waves issued theirs; the
    // exchange wave first reads the shared slot (a poll issued after weight
    // loads would wait for them)
    wait_lds(&s_dissued, (uint32_t)kGuWaves);
    const int eo = __builtin_amdgcn_readfirstlane(s_ids[ks]);
    const bool oko = eo >= 0 && eo < a.E;
    const float wko = oko ? s_w[ks] : 0.f;
    if (xchg && a.has_shared) exchange_until(K, 0);
    {
      // an invalid id reads expert 0 and contributes 0
      const __amdgpu_buffer_rsrc_t rs = blob_rsrc(a.experts + (size_t)(oko ? eo : 0) * a.stride);
#pragma unroll
      for (int ld = 0; ld < Gm::RDLD; ++ld) {
        const int row = obase + ld * Gm::RPL + lane / Gm::LPR;
        dqr[ld] = ld_codes(rs, row);
        dsbr[ld] = bld4(rs, o_dsb(row));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // shared rows (lane partial sums, one per row)
    float accs[Gm::DLD];
#pragma unroll
    for (int ld = 0; ld < Gm::DLD; ++ld) accs[ld] = 0.f;
    if (a.has_shared) {
      if (!xchg) wait_lds(&s_hready[0], 1u);
      down_rows<BITS, Gm::DLD, Gm::DWORDS, Gm::DCOLS>(dqs, dsbs, &s_hb[0][seg * Gm::DCOLS],
                                                      hb_key(seg), 1.f, accs);
    }
    // own routed rows, then their sums to the workgroups that own the rows:
    // lane 2 ld + j of the wave stores row obase + 2 ld + j
    if (xchg) exchange_until(ks, 1);
    else wait_lds(&s_hready[1], 1u);
    {
      float acco[Gm::RDLD];
#pragma unroll
      for (int ld = 0; ld < Gm::RDLD; ++ld) acco[ld] = 0.f;
      down_rows<BITS, Gm::RDLD, Gm::DWORDS, Gm::DCOLS>(dqr, dsbr, &s_hb[1][seg * Gm::DCOLS],
                                                       hb_key(seg), wko, acco);
      static_assert(Gm::RPL == 2 && Gm::LPR == 32, "two rows per wave-wide load");
      float pv = 0.f;
#pragma unroll
      for (int ld = 0; ld < Gm::RDLD; ++ld) {
        float lo, hi;
        half_sums32(acco[ld], lo, hi);
        pv = lane == 2 * ld ? lo : pv;
        pv = lane == 2 * ld + 1 ? hi : pv;
      }
      if (lane < Gm::O_ROWS_W) {
        const uint64_t v = ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(pv);
        __hip_atomic_store(&a.ptag[(size_t)ks * H + obase + lane], v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (xchg) {
      // the routed sums can only be complete once every workgroup published
      // every slot, this one included
      while (true) {
        count_published();
        if (published == K && try_parts()) break;
        if (timed_out()) {
          if (lane == 0) *lds(&s_pready) = 1u;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    } else {
      wait_lds(&s_pready, 1u);
    }
    // y = shared + routed sums of slots 0 .. K-1, in that order
#pragma unroll
    for (int ld = 0; ld < Gm::DLD; ++ld) {
      float v = lane_group_sum<Gm::LPR>(accs[ld], lane);
      const int i = rows[ld] - b * Gm::D_ROWS;
#pragma unroll
      for (int k = 0; k < K; ++k) v += s_part[k][i];
      if (seg == 0) {
        if (!RES || a.y) a.y[rows[ld]] = v;
        if (RES) a.resid[rows[ld]] = rres[ld] + v;
      }
    }
    // this workgroup has read activations of every workgroup, published after
    // barrier (A), where they read the epoch
    if (b == 0 && xchg && lane < kGroups)
      __hip_atomic_store(&a.fc->epoch[lane][0], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Dequantisation hook of the fp8 pair convert: s q + z per code, with q the
// value fp8_word_codes forms (u q) times 1 / u (exact, a power of two).
template <int BITS>
__global__ void __launch_bounds__(256) k_dequant_fp8(DequantArgs a) {
  constexpr int CPW = 32 / BITS;
  uint32_t m = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  asm volatile("" : "+s"(m));
  const float iu = 1.f / fp8_code_unit();
  const int wpr = a.cols / CPW;
  const size_t n = (size_t)a.rows * wpr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / wpr;
    const int c0 = (int)(i - r * wpr) * CPW;
    float q[CPW];
    fp8_word_codes<BITS>(a.q[i], m, q);
#pragma unroll
    for (int j = 0; j < CPW; ++j) q[j] *= iu;
    store_dequant_word<CPW>(a, r, c0, q);
  }
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_dequant_fp8(const DequantArgs &a, int blocks, void *stream) {
  if (a.bits == 4)
    hipLaunchKernelGGL(k_dequant_fp8<4>, dim3(blocks), dim3(256), 0, S(stream), a);
  else
    hipLaunchKernelGGL(k_dequant_fp8<2>, dim3(blocks), dim3(256), 0, S(stream), a);
  return (int)hipGetLastError();
}

// Returns true if the fused single-token kernel covers these dims.
bool fused_supported(const moe_dims &d) {
  static int ncu = -1;
  if (ncu < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 0;
  }
  return ncu == kG && d.hidden == 4096 && d.inter == 1024 && d.top_k == 4 &&
         (d.bits == 4 || d.bits == 2);
}

int launch_layer_fused(const moe_dims &d, const moe_layer &L, const uint16_t *x,
                       const int32_t *ids_in, const float *w_in, int32_t *ids_out,
                       float *w_out, float *y, float *resid, uint16_t *x_out, void *ws,
                       void *stream) {
  const WsLayout W = ws_layout(d, 1);
  const BlobLayout B = blob_layout(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  FusedArgs a;
  a.x = x;
  a.router = L.router;
  a.experts = L.experts;
  a.shared = L.shared;
  a.stride = L.expert_stride;
  a.ids_in = ids_in;
  a.w_in = w_in;
  a.ids_out = ids_out;
  a.w_out = w_out;
  a.y = y;
  a.resid = resid;
  a.x_out = x_out;
  a.ctrl = reinterpret_cast<Ctrl *>(base + W.ctrl);
  a.fc = reinterpret_cast<FCtrl *>(base + W.fctrl);
  a.tags = reinterpret_cast<uint64_t *>(base + W.logits_tag);
  a.htag = reinterpret_cast<uint64_t *>(base + W.h_tag);
  a.ptag = reinterpret_cast<uint64_t *>(base + W.p_tag);
  a.E = d.n_experts;
  a.has_shared = d.has_shared;
  a.off_gq = (int64_t)B.off[MOE_SEC_GATE_Q];
  a.off_uq = (int64_t)B.off[MOE_SEC_UP_Q];
  a.off_dq = (int64_t)B.off[MOE_SEC_DOWN_Q];
  a.off_gsb = (int64_t)B.off[MOE_SEC_GATE_SB];
  a.off_usb = (int64_t)B.off[MOE_SEC_UP_SB];
  a.off_dsb = (int64_t)B.off[MOE_SEC_DOWN_SB];
  const int rr = (d.n_experts + kG - 1) / kG;
  // the residual mode always routes
  if (resid && ids_in) return (int)hipErrorInvalidValue;
#define MOE_LAUNCH_L1(B, R, RS) \
  hipLaunchKernelGGL((k_layer1<B, 4096, 1024, 4, R, RS>), dim3(kG), dim3(kNT), 0, S(stream), a)
#define MOE_LAUNCH_RR(B, RS)        \
  if (rr == 1) MOE_LAUNCH_L1(B, 1, RS); \
  else if (rr == 2) MOE_LAUNCH_L1(B, 2, RS); \
  else MOE_LAUNCH_L1(B, 4, RS)
  if (d.bits == 4) {
    if (resid) { MOE_LAUNCH_RR(4, true); } else { MOE_LAUNCH_RR(4, false); }
  } else {
    if (resid) { MOE_LAUNCH_RR(2, true); } else { MOE_LAUNCH_RR(2, false); }
  }
#undef MOE_LAUNCH_RR
#undef MOE_LAUNCH_L1
  return (int)hipGetLastError();
}

}  // namespace moe
