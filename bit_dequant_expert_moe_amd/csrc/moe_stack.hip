// moe_stack.hip -- consecutive MoE layers of one decode token in one launch.
//
// Method: "Flash-MoE: Running a 397B Parameter Model on a Laptop"
// (hysenlabs.com), section "How the SSD expert streaming pipeline works":
// per layer, router -> softmax + top-K -> expert forward of the K selected
// experts and the shared expert -> combine (and, on the residual stream, a
// norm before the next layer's router); the next layer's command is already
// queued while the current one runs, so the GPU does not wait between
// layers.  "Flash-MoE: Running a 400 Billion Parameter Model on a MacBook"
// (mattcullerton.com), section "The Architecture": 4-bit experts
// dequantised inside the FMA inner loop.
//
// This kernel runs the per-layer work of k_layer1 (moe_fused.hip; the same
// 256 resident workgroups, wave roles and one-way tagged exchanges) for L
// layers in a loop, so that:
//   * there is no kernel boundary between layers (each launch of a layer
//     drains the GPU and ramps up again, ~2 us per layer);
//   * the bytes of layer l+1 that do not depend on its routing -- its router
//     rows (4 MB), its x (plain mode) and its shared expert's gate/up rows
//     (4.7 MB) -- are requested by the gate/up waves right after they have
//     computed layer l's shared expert, and arrive while layer l's logits
//     exchange keeps HBM otherwise idle.
// A layer's dependent work still waits for the layer before it: a workgroup
// publishes layer l+1's logits only after it has finished layer l, and on
// the residual stream x of layer l+1 is the norm of r + y, gathered from all
// workgroups once every one of them has formed its rows of y.
//
// The arithmetic of every result (router sums, top-K and weights, gate/up
// and down products, the combine, the norm) is the one k_layer1 performs, in
// the same order: the ids, weights and outputs of a layer are bitwise those
// of a moe_layer_decode (or moe_layer_decode_residual) call on the same
// inputs.  The router rows sit in the gate/up waves (two x chunks per
// thread); their partial sums are reduced as the eight waves of k_layer1
// reduce them.
//
// Per-layer exchange epochs: layer l of a launch carries epoch base + 1 + l,
// base = the epoch of the last completed call on the workspace.  A workgroup
// writes an exchange word of layer l+1 only after it has read every word of
// layer l that any workgroup needs from that array (it has passed layer l's
// routing, which needs every workgroup's layer-l logits, and so on), so one
// copy of each array serves all layers.
//
// Residual stream (RES): the row owners keep their 16 rows of r in
// registers; at the end of each layer they store r + y as tagged words (one
// copy per reader group); every workgroup gathers the 4096 words of the
// layer before it, then forms x = bf16(r / rms(r)) exactly as k_layer1 does
// (each of the 512 threads its 8 columns, the sum of squares reduced in wave
// order).  The last layer writes r back to the caller's buffer.
//
// Polls read two 8-byte tagged words with one 16-byte load; they rely on the
// load returning each aligned 8-byte half as written by a single 8-byte
// store (no mix of two stores inside one half), which holds for 16-byte
// aligned vector loads on this GPU (the memory system moves whole 32-byte
// sectors) but is not stated by the HIP memory model.
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

struct StackLayer {
  const uint16_t *router;
  const uint8_t *experts, *shared;
  int64_t stride;
};

struct StackArgs {
  StackLayer L[kMaxStackLayers];
  int n_layers;
  const uint16_t *x;  // plain mode: bf16 [n_layers][H]
  float *y;           // fp32 [n_layers][H] (plain mode) or null (residual mode)
  int32_t *ids_out;   // [n_layers][K] or null
  float *w_out;       // [n_layers][K] or null
  float *resid;       // residual mode: r, fp32 [H], read at the start, written at the end
  uint16_t *x_out;    // residual mode: bf16 [n_layers][H] or null
  Ctrl *ctrl;
  FCtrl *fc;
  uint64_t *tags;  // [kGroups][kMaxE] tagged logits
  uint64_t *htag;  // [kGroups][K+1][I] tagged activations
  uint64_t *rtag;   // residual mode: [kGroups][H] tagged r + y
  uint64_t *rdone;  // residual mode: [kGroups][kG] tagged: the workgroup's rows are stored
  int E, has_shared;
  int64_t off_gq, off_uq, off_dq, off_gsb, off_usb, off_dsb;
};

// Timestamps of the layer's steps, per workgroup, for a build with
// MOE_STACK_TRACE defined (the trace buffer's device address sits in the
// workspace control block); empty otherwise.
// They are kept in LDS and copied out when the kernel ends, so that taking
// them adds no global store for a later wait on the vector memory counter.
#ifdef MOE_STACK_TRACE
constexpr int kTrEv = 48;  // events per (workgroup, layer)
#define MOE_TRACE(ev)                                                          \
  do {                                                                         \
    if (lane == 0) s_tr[l * kTrEv + (ev)] = __builtin_amdgcn_s_memrealtime();  \
  } while (0)
#else
#define MOE_TRACE(ev) \
  do {                \
  } while (0)
#endif

// Which rows of each matrix a workgroup owns: 0 a contiguous block (rows
// b n .. b n + n - 1), 1 every 256th row from b (rows b, b + 256, ...), which
// spreads each workgroup's bytes over the whole matrix.
#ifndef MOE_STACK_ILV
#define MOE_STACK_ILV 0
#endif

// When the gate/up waves request the next layer's routing-independent bytes:
// 0 right after the shared expert's gate/up products (during the logits
// exchange), 1 right after the routed loads, 2 after the routed products,
// 3 in four parts, one after each routed slot's products.
#ifndef MOE_STACK_PF
#define MOE_STACK_PF 3
#endif

// When the down-row waves issue their routed rows' loads: -1 as soon as the
// gate/up waves have issued theirs, k >= 0 once this workgroup has
// published its activations of routed slot k.
#ifndef MOE_STACK_RDELAY
#define MOE_STACK_RDELAY 0
#endif

// When the down-row waves load the next layer's shared-expert rows: 0 at the
// start of that layer (just before its routing), 1 as soon as they have
// computed the current layer's shared rows (their registers are free then),
// so that those loads are not in the memory pipeline when the logits poll
// of the next layer is issued (measured: no faster).
#ifndef MOE_STACK_RPF
#define MOE_STACK_RPF 0
#endif

// Copies of every exchanged datum (logits, activations, r + y, done words):
// a reader reads copy b % kCopies, a writer stores into all of them.  The
// workgroups b with the same b % 8 share an XCD (and its L2).
#ifndef MOE_STACK_COPIES
#define MOE_STACK_COPIES 8
#endif
constexpr int kCopies = MOE_STACK_COPIES;
static_assert(kCopies >= 1 && kCopies <= kGroups && kGroups % kCopies == 0, "copies");

// Polls in flight and their spacing (sleep units of 64 clocks) of the
// exchange wave's three waits: every workgroup's logits, one slot's
// activations, and (residual mode) every workgroup's done word.
// (Measured: one poll at a time is fastest.  With more in flight, a poll
// that succeeds waits for the later ones before their registers are reused,
// and the extra coherent reads of the same lines slow every poll.)
#ifndef MOE_STACK_LOGIT_POLLS
#define MOE_STACK_LOGIT_POLLS 1
#endif
#ifndef MOE_STACK_H_POLLS
#define MOE_STACK_H_POLLS 1
#endif
#ifndef MOE_STACK_R_POLLS
#define MOE_STACK_R_POLLS 1
#endif
#ifndef MOE_STACK_POLL_GAP
#define MOE_STACK_POLL_GAP 8
#endif

// A layer's pointers read from LDS, made wave-uniform (scalar registers), so
// that the buffer resources built from them stay scalar (from vector
// registers every buffer load would need a loop over the lanes' values).
// (readfirstlane returns a signed int: each half goes through uint32_t, or
// the low half's sign would spread into the high word)
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ StackLayer uniform_layer(const StackLayer &s) {
  StackLayer r;
  r.router = reinterpret_cast<const uint16_t *>(uniform64(reinterpret_cast<uint64_t>(s.router)));
  r.experts = reinterpret_cast<const uint8_t *>(uniform64(reinterpret_cast<uint64_t>(s.experts)));
  r.shared = reinterpret_cast<const uint8_t *>(uniform64(reinterpret_cast<uint64_t>(s.shared)));
  r.stride = (int64_t)uniform64((uint64_t)s.stride);
  return r;
}

// Which weight loads carry the non-temporal hint: 0 none, 1 the routed
// experts', 2 also the shared expert's and the router's.
#ifndef MOE_STACK_NT
#define MOE_STACK_NT 1
#endif
constexpr int kPolRouted = MOE_STACK_NT >= 1 ? kPolStream : 0;
// First wait of the exchange wave before its logits poll, in s_sleep units
// (64 clocks): a poll issued before the last logits can be visible comes
// back incomplete and costs a whole round trip.
#ifndef MOE_STACK_SLEEP0
#define MOE_STACK_SLEEP0 19
#endif
constexpr int kPolShared = MOE_STACK_NT >= 2 ? kPolStream : 0;

// LDS-only workgroup barrier: orders the waves' LDS accesses without waiting
// for their global loads in flight (a barrier with a global fence would wait
// for the prefetched weights).
__device__ __forceinline__ void lds_barrier() {
  lds_release();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
}

template <int BITS, int H, int I, int K, int RR, bool RES>
__global__ void __launch_bounds__(kNT, 1) k_stack(StackArgs a) {
  using Gm = Geo<BITS, H, I, K>;
  constexpr int COLS = Gm::COLS, PAIRS = Gm::PAIRS, LSEG = Gm::LSEG;
  constexpr int NSL = K + 1;   // slot K is the shared expert
  constexpr int NW = kNT / 64;  // waves; the router and the norm reduce in their order
  static_assert(NSL == kFusedSlots && I == kFusedI && H == kFusedH, "exchange arrays' sizes");
  static_assert(Gm::RXC == 1, "one 8-column x chunk per thread of the workgroup");
  static_assert(NW == 2 * kGuWaves, "the gate/up waves hold the router chunks of two waves");
  static_assert(MOE_STACK_PF != 3 || K == 4, "four prefetch parts, one per routed slot");
  __shared__ float s_red[NW][RR];
  __shared__ uint32_t s_xp[2][Gm::SEG_X][PAIRS];  // packed x pairs, by layer parity
  __shared__ float2 s_cx[2][Gm::SEG_X];           // (1024 * sum of pairs, sum of x)
  __shared__ float s_hb[NSL][I];                  // h of every slot
  __shared__ int32_t s_ids[K];
  __shared__ float s_w[K];
  __shared__ uint32_t s_cnt[NSL];     // gate/up rows published per slot, over all layers so far
  __shared__ uint32_t s_hready[NSL];  // layers whose s_hb[slot] is filled
  __shared__ uint32_t s_epoch;        // epoch of the last call completed before this one
  __shared__ uint32_t s_ready;        // layers routed
  __shared__ uint32_t s_gu_issued;    // gate/up waves x layers whose routed loads are issued
  __shared__ float s_ss[NW];          // residual mode: sum of r^2 per wave
  __shared__ uint4 s_xn[RES ? H / 8 : 1];  // residual mode: normalised x, bf16
  __shared__ uint32_t s_rseen;        // residual mode: layers whose r + y words are all written
  __shared__ uint32_t s_rstored;      // residual mode: row waves x layers that stored their r + y
  // the layers' pointers, copied from the kernel arguments once (a scalar
  // load of a later layer's entry from the argument segment can miss the
  // scalar cache and cost a memory round trip on the routing path)
  __shared__ StackLayer s_L[kMaxStackLayers];
#ifdef MOE_STACK_TRACE
  __shared__ uint64_t s_tr[kMaxStackLayers * kTrEv];
#endif

  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = b % kCopies;  // the exchange copy this workgroup reads
  const int NL = a.n_layers;
  constexpr int rr = RR;  // router rows per workgroup (E <= RR * kG)

#ifdef MOE_STACK_TRACE
  uint64_t *trace = *reinterpret_cast<uint64_t *const *>(&a.ctrl->pad[0]);
  for (int i = tid; i < kMaxStackLayers * kTrEv; i += kNT) s_tr[i] = 0;
#endif
  // the router row `row` of this workgroup (an expert index)
  auto router_row = [&](int row) -> int { return MOE_STACK_ILV ? row * kG + b : b * RR + row; };
  constexpr int kEpochTid = kNT - 64;
  uint32_t epoch_done = (uint32_t)a.E;
  if (tid == kEpochTid) epoch_done = ld_rlx(&a.fc->epoch[b % kGroups][0]);
  if (tid < NSL) {
    s_cnt[tid] = 0u;
    s_hready[tid] = 0u;
  }
  if (tid == 0) {
    s_ready = 0u;
    s_gu_issued = 0u;
    s_rseen = 0u;
    s_rstored = 0u;
  }
  static_assert(sizeof(StackLayer) == 32, "four 8-byte words per layer");
  if (tid < 4 * NL)
    reinterpret_cast<uint64_t *>(s_L)[tid] = reinterpret_cast<const uint64_t *>(a.L)[tid];
  lds_barrier();

  // ---- residual mode: r of this thread's chunk (8 columns) and the norm ----
  // layer 0 reads the caller's r; layer l > 0 gathers r + y of layer l-1
  // from the row owners' tagged words (this group's copy)
  float4 rf[2];  // (used in residual mode only)
  uint4 rx_own;  // bf16 x of chunk tid (residual mode)
  auto gather_r = [&](int l, uint32_t epoch_prev) {
    if (l == 0) {
      const float4 *p = reinterpret_cast<const float4 *>(a.resid + (size_t)tid * 8);
      rf[0] = p[0];
      rf[1] = p[1];
      return;
    }
    // the exchange wave polls the dense array of the writers' done words
    // (2 KB) until all carry the previous layer's epoch; then every thread
    // reads its 8 words once (again only if one of them is still old: a done
    // word orders nothing, the tags of the data words decide)
    if (wave == kGuWaves) {
      long spins = 0;
      const uint32_t base = (uint32_t)((size_t)grp * kG * 8);
      constexpr int NWD = kG / 128;
      const bool done = poll_pipe<MOE_STACK_R_POLLS, 8, MOE_STACK_POLL_GAP, NWD>(
          [&](uint4 (&u)[NWD]) {
#pragma unroll
            for (int i = 0; i < NWD; ++i)
              u[i] = ld_coh16(a.rdone, base + (uint32_t)(128 * i + 2 * lane) * 8u);
          },
          [&](const uint4 (&u)[NWD]) {
            bool ok = true;
#pragma unroll
            for (int i = 0; i < NWD; ++i) ok &= u[i].y == epoch_prev && u[i].w == epoch_prev;
            return __all(ok) != 0;
          },
          [&](const uint4 (&)[NWD]) {}, spins);
      if (!done && lane == 0) atomicOr(&a.ctrl->err, 2u);
      lds_release();
      if (lane == 0) *lds(&s_rseen) = (uint32_t)l;
    }
    wait_lds(&s_rseen, (uint32_t)l);
    const uint32_t base = (uint32_t)(((size_t)grp * H + (size_t)tid * 8) * 8);
    long spins = 0;
    while (true) {
      uint4 t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = ld_coh16(a.rtag, base + 16u * i);
      bool ok = true;
#pragma unroll
      for (int i = 0; i < 4; ++i) ok &= t[i].y == epoch_prev && t[i].w == epoch_prev;
      if (__all(ok) || ++spins > kSpinMax) {
        if (!__all(ok) && lane == 0) atomicOr(&a.ctrl->err, 2u);
        rf[0] = make_float4(__uint_as_float(t[0].x), __uint_as_float(t[0].z),
                            __uint_as_float(t[1].x), __uint_as_float(t[1].z));
        rf[1] = make_float4(__uint_as_float(t[2].x), __uint_as_float(t[2].z),
                            __uint_as_float(t[3].x), __uint_as_float(t[3].z));
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  // x = bf16(r / sqrt(mean(r^2) + eps)) into rx_own and s_xn: the per-wave
  // sums are added in wave order, so every workgroup uses the same scale
  // (the arithmetic of k_layer1's residual mode)
  auto norm_x = [&](int l) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ss = fmaf(rf[j].x, rf[j].x, ss);
      ss = fmaf(rf[j].y, rf[j].y, ss);
      ss = fmaf(rf[j].z, rf[j].z, ss);
      ss = fmaf(rf[j].w, rf[j].w, ss);
    }
    ss = wave_sum64(ss);
    if (lane == 0) s_ss[wave] = ss;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_ss[w];
    const float inv = 1.f / sqrtf(tot * (1.f / (float)H) + kRmsEps);
    const float4 lo = rf[0], hi = rf[1];
    rx_own = make_uint4(f2bf(lo.x * inv) | (f2bf(lo.y * inv) << 16),
                        f2bf(lo.z * inv) | (f2bf(lo.w * inv) << 16),
                        f2bf(hi.x * inv) | (f2bf(hi.y * inv) << 16),
                        f2bf(hi.z * inv) | (f2bf(hi.w * inv) << 16));
    s_xn[tid] = rx_own;
    if (b == 0 && a.x_out)
      *reinterpret_cast<uint4 *>(a.x_out + (size_t)l * H + (size_t)tid * 8) = rx_own;
    lds_barrier();
  };

  if (wave < kGuWaves) {
    // ========================= gate/up waves ================================
    // thread t holds the router rows' chunks t and t + kNT / 2 (x columns
    // 8 t .. 8 t + 7 and the same 2048 columns further), i.e. the chunks of
    // the threads t of waves `wave` and `wave + 4` of k_layer1
    // this wave's row of every slot
    const int r = MOE_STACK_ILV ? wave * kG + b : b * Gm::GU_ROWS + wave;
    const size_t rbytes = (size_t)H * BITS / 8;
    const int groups = H / kGroup;
    const int xs = tid;  // x segment staged by this thread (if < SEG_X)
    constexpr int HALF = kNT / 2;
    uint4 gq[NSL][LSEG], uq[NSL][LSEG];
    uint32_t gsb[NSL][LSEG], usb[NSL][LSEG];
    uint4 rw[RR][2], rx2[2], xr[Gm::XLD];
    uint32_t o_gq[LSEG], o_uq[LSEG], o_gsb[LSEG], o_usb[LSEG];
#pragma unroll
    for (int j = 0; j < LSEG; ++j) {
      const int sg = lane + 64 * j;
      o_gq[j] = (uint32_t)(a.off_gq + (int64_t)r * rbytes + sg * 16);
      o_uq[j] = (uint32_t)(a.off_uq + (int64_t)r * rbytes + sg * 16);
      o_gsb[j] = (uint32_t)(a.off_gsb + ((int64_t)r * groups + sg * COLS / kGroup) * 4);
      o_usb[j] = (uint32_t)(a.off_usb + ((int64_t)r * groups + sg * COLS / kGroup) * 4);
    }
    auto load_rows = [&](auto pol_tag, int slot, const uint8_t *bl) {
      constexpr int P = decltype(pol_tag)::value;
      const __amdgpu_buffer_rsrc_t rs = blob_rsrc(bl);
#pragma unroll
      for (int j = 0; j < LSEG; ++j) {
        gq[slot][j] = bld16<P>(rs, o_gq[j]);
        uq[slot][j] = bld16<P>(rs, o_uq[j]);
        gsb[slot][j] = bld4<P>(rs, o_gsb[j]);
        usb[slot][j] = bld4<P>(rs, o_usb[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // the bytes of layer l that do not depend on its routing
    // (router rows and x through buffer resources: a load through a generic
    // pointer is a FLAT load, which also counts on the LDS counter, so the
    // next LDS read would wait for it)
    auto load_router = [&](const StackLayer &Ly) {
      const __amdgpu_buffer_rsrc_t rr_rs =
          blob_rsrc(reinterpret_cast<const uint8_t *>(Ly.router));
#pragma unroll
      for (int row = 0; row < RR; ++row) {
        const int e = router_row(row);
        // rows past E read row E-1 and are never published
        const int ec = e < a.E ? e : a.E - 1;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          rw[row][c] = bld16<kPolShared>(rr_rs, (uint32_t)(((size_t)ec * H +
                                                            (size_t)(tid + HALF * c) * 8) * 2));
      }
    };
    auto load_x = [&](int l) {
      const __amdgpu_buffer_rsrc_t x_rs = blob_rsrc(reinterpret_cast<const uint8_t *>(a.x));
      const uint32_t xo = (uint32_t)((size_t)l * H * 2);
#pragma unroll
      for (int c = 0; c < 2; ++c) rx2[c] = bld16(x_rs, xo + (uint32_t)((tid + HALF * c) * 16));
#pragma unroll
      for (int t = 0; t < Gm::XLD; ++t)
        xr[t] = bld16(x_rs, xo + (uint32_t)(((xs % Gm::SEG_X) * COLS + 8 * t) * 2));
    };
    // the bytes of layer l that do not depend on its routing
    auto prefetch = [&](int l) {
      const StackLayer Ly = uniform_layer(s_L[l]);
      load_router(Ly);
      if (!RES) load_x(l);
      // without a shared expert slot K reads expert 0 and is never used
      load_rows(std::integral_constant<int, kPolShared>{}, K, a.has_shared ? Ly.shared : Ly.experts);
    };
    // the same bytes in four parts (MOE_STACK_PF 3: one part after each routed
    // slot's products, so that little of it is queued ahead of a poll)
    auto prefetch_part = [&](int l, int part) {
      const StackLayer Ly = uniform_layer(s_L[l]);
      if (part == 0) {
        load_router(Ly);
        return;
      }
      const __amdgpu_buffer_rsrc_t rs = blob_rsrc(a.has_shared ? Ly.shared : Ly.experts);
      if (part == 1) {
        if (!RES) load_x(l);
#pragma unroll
        for (int j = 0; j < LSEG; ++j) gq[K][j] = bld16<kPolShared>(rs, o_gq[j]);
      } else if (part == 2) {
#pragma unroll
        for (int j = 0; j < LSEG; ++j) uq[K][j] = bld16<kPolShared>(rs, o_uq[j]);
      } else {
#pragma unroll
        for (int j = 0; j < LSEG; ++j) {
          gsb[K][j] = bld4<kPolShared>(rs, o_gsb[j]);
          usb[K][j] = bld4<kPolShared>(rs, o_usb[j]);
        }
      }
    };
    prefetch(0);

    for (int l = 0; l < NL; ++l) {
      const StackLayer Ly = uniform_layer(s_L[l]);
      const int buf = l & 1;
      if (RES) {
        gather_r(l, s_epoch + (uint32_t)l);  // (s_epoch is read only for l > 0)
        if (wave == 0) MOE_TRACE(27);
        norm_x(l);
        if (wave == 0) MOE_TRACE(28);
        rx2[0] = rx_own;
        rx2[1] = s_xn[tid + HALF];
#pragma unroll
        for (int t = 0; t < Gm::XLD; ++t) xr[t] = s_xn[(xs % Gm::SEG_X) * (COLS / 8) + t];
        if (wave == 0) MOE_TRACE(30);
      }
      // router partials, reduced as k_layer1's waves `wave` and `wave + 4`
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int row = 0; row < RR; ++row) {
          const uint4 wv = rw[row][c], xv = rx2[c];
          float acc = 0.f;
          acc = dot2b(wv.x, xv.x, acc);
          acc = dot2b(wv.y, xv.y, acc);
          acc = dot2b(wv.z, xv.z, acc);
          acc = dot2b(wv.w, xv.w, acc);
          const float v = wave_sum64(acc);
          if (lane == 0) s_red[wave + kGuWaves * c][row] = v;
        }
      }
      if (wave == 0) MOE_TRACE(31);
      // x pairs and per-segment corrections, one code word at a time, to LDS
      if (xs < Gm::SEG_X) {
        float C = 0.f, X = 0.f;
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(&xr[0]);
        const int xkey = xp_key<PAIRS>(xs);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          constexpr int CPW = 32 / BITS;
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
              s_xp[buf][xs][(4 * wd + p) ^ xkey] = pr;
              C += h2_sum(pr);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int e = k < 5 ? k : k - 5;
              const float sc = 1.f / (float)(1 << (2 * e));
              const uint32_t pr = pack_h2(v[k] * sc, v[k + 8] * sc);
              s_xp[buf][xs][(8 * wd + k) ^ xkey] = pr;
              C += h2_sum(pr);
            }
          }
        }
        s_cx[buf][xs] = make_float2(1024.f * C, X);
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
            const uint4 q = *reinterpret_cast<const uint4 *>(&s_xp[buf][sg][p ^ xk]);
            xp[p] = q.x;
            xp[p + 1] = q.y;
            xp[p + 2] = q.z;
            xp[p + 3] = q.w;
          }
          const float2 cx = s_cx[buf][sg];
          const float ag = seg_dot_x<BITS>(gq[slot][j], xp) - cx.x;
          const float au = seg_dot_x<BITS>(uq[slot][j], xp) - cx.x;
          pg += bf16f(gsb[slot][j] & 0xFFFFu) * ag + bf16f(gsb[slot][j] >> 16) * cx.y;
          pu += bf16f(usb[slot][j] & 0xFFFFu) * au + bf16f(usb[slot][j] >> 16) * cx.y;
        }
        pg = wave_sum64(pg);
        pu = wave_sum64(pu);
        return pg / (1.f + expf(-pg)) * pu;
      };
      if (wave == 0) MOE_TRACE(29);
      lds_barrier();  // (A) router partials, x pairs, epoch
      if (wave == 0) MOE_TRACE(8);
      const uint32_t epoch = s_epoch + 1u + (uint32_t)l;
      auto publish = [&](int slot, float hv) {
        if (lane < kCopies)
          __hip_atomic_store(&a.htag[((size_t)lane * NSL + slot) * I + r],
                             ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(hv),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0)
          __hip_atomic_fetch_add(&s_cnt[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      };
      if (a.has_shared) publish(K, gateup(K));
      if (wave == 0) MOE_TRACE(9);
      // layer l+1's router rows, x and shared gate/up rows (slot K's
      // registers are free now)
      if (MOE_STACK_PF == 0 && l + 1 < NL) prefetch(l + 1);
      wait_lds(&s_ready, (uint32_t)(l + 1));
      int eid[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        eid[k] = __builtin_amdgcn_readfirstlane(s_ids[k]);
        const bool ok = eid[k] >= 0 && eid[k] < a.E;
        // an invalid id reads expert 0 and contributes 0
        load_rows(std::integral_constant<int, kPolRouted>{}, k,
                  Ly.experts + (size_t)(ok ? eid[k] : 0) * Ly.stride);
      }
      // the down rows' loads go after these (the activations, which every
      // down row waits for, come from these bytes)
      if (lane == 0)
        __hip_atomic_fetch_add(&s_gu_issued, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (MOE_STACK_PF == 1 && l + 1 < NL) prefetch(l + 1);
      if (wave == 0) MOE_TRACE(10);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const bool ok = eid[k] >= 0 && eid[k] < a.E;
        publish(k, ok ? gateup(k) : 0.f);
        if (wave == 0 && k < 4) MOE_TRACE(11 + k);
        // (issued on the last layer too, again for that layer: a load under
        // a condition makes the compiler's later waits count conservatively)
        if (MOE_STACK_PF == 3) prefetch_part(l + 1 < NL ? l + 1 : l, k);
      }
      if (MOE_STACK_PF == 2 && l + 1 < NL) prefetch(l + 1);
    }
  } else if (wave == kGuWaves) {
    // ========================= exchange wave ================================
    // Reads what the workgroup needs from the other workgroups, into LDS:
    // every workgroup's logits (then selects the top-K), and the activations
    // h of every slot (the shared one, then routed slots 0 .. K-1 as each is
    // complete everywhere).  It loads no weights, so no poll of it waits for
    // a weight load.
    for (int l = 0; l < NL; ++l) {
      if (RES) {
        gather_r(l, l == 0 ? 0u : s_epoch + (uint32_t)l);
        MOE_TRACE(15);
        norm_x(l);
      }
      if (l == 0 && tid == kEpochTid) s_epoch = epoch_done;
      lds_barrier();  // (A)
      MOE_TRACE(0);
      const uint32_t epoch = s_epoch + 1u + (uint32_t)l;
      const uint32_t want = (uint32_t)(l + 1);  // LDS flag value of this layer
      long xspins = 0;  // one poll budget per layer
      // 1. (this workgroup's logits are published by the last down-row
      //    wave: this wave issues no stores, since a later wait of its
      //    memory counter would also wait for a store's acknowledgement)
      // 2. routing: every workgroup's logits of this layer in this group's
      //    copy, then the top-K (the selection is deterministic, so all
      //    workgroups agree)
      {
        const uint64_t *tags_mine = a.tags + (size_t)grp * kMaxE;
        constexpr int NV = 4 * RR;
        static_assert(256 * RR <= kMaxE, "tag copy holds 256 RR entries");
        float v[NV];
        __builtin_amdgcn_s_sleep(MOE_STACK_SLEEP0);
#ifdef MOE_STACK_TRACE
        int npoll = 0;
#endif
        const bool done = poll_pipe<MOE_STACK_LOGIT_POLLS, 8, MOE_STACK_POLL_GAP, NV / 2>(
            [&](uint4 (&t)[NV / 2]) {
#pragma unroll
              for (int i = 0; i < NV / 2; ++i)
                t[i] = ld_coh16(tags_mine, (uint32_t)(128 * i + 2 * lane) * 8u);
#ifdef MOE_STACK_TRACE
              if (npoll++ == 0) MOE_TRACE(25);
              if (lane == 0) s_tr[l * kTrEv + 26] = (uint64_t)npoll * 100;
#endif
            },
            [&](const uint4 (&t)[NV / 2]) {
#ifdef MOE_STACK_TRACE
              if (npoll == 1) MOE_TRACE(5);
#endif
              bool ok = true;
#pragma unroll
              for (int i = 0; i < NV / 2; ++i) {
                const int idx = 128 * i + 2 * lane;
                ok &= (idx >= a.E || t[i].y == epoch) && (idx + 1 >= a.E || t[i].w == epoch);
              }
              return __all(ok) != 0;
            },
            [&](const uint4 (&t)[NV / 2]) {
#pragma unroll
              for (int i = 0; i < NV / 2; ++i) {
                const int idx = 128 * i + 2 * lane;
                v[2 * i] = idx < a.E ? __uint_as_float(t[i].x) : __builtin_nanf("");
                v[2 * i + 1] = idx + 1 < a.E ? __uint_as_float(t[i].z) : __builtin_nanf("");
              }
            },
            xspins);
        if (!done && lane == 0) atomicOr(&a.ctrl->err, 2u);
        MOE_TRACE(34);
        float sel_v[K];
        int sel_i[K];
        topk_select<K, NV>(v, lane, sel_v, sel_i);
        MOE_TRACE(32);
        int id;
        float wk;
        topk_weights<K>(sel_v, sel_i, lane, id, wk);
        if (lane < K) {
          s_ids[lane] = id;
          s_w[lane] = wk;
        }
      }
      // 3. activations h from this group's copy into s_hb: a slot is complete
      //    once every entry carries this layer's epoch.  A poll waits behind
      //    every load this CU has issued before it, so the shared slot's poll
      //    is issued before the routing is handed to the other waves (their
      //    routed loads then queue behind it), and the routed slots are read
      //    in rounds: each round polls every slot that this workgroup has
      //    published its own rows of (the others publish at about the same
      //    time) and that is not read yet.
      constexpr int NLD = I / 128;  // 16-byte loads per lane (two entries each)
      auto h_issue = [&](int slot, uint4 (&t)[NLD]) {
        const uint32_t base = (uint32_t)(((size_t)grp * NSL + slot) * I * 8);
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          t[i] = ld_coh16(a.htag, base + (uint32_t)(128 * i + 2 * lane) * 8u);
      };
      auto h_ok = [&](const uint4 (&t)[NLD]) -> bool {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NLD; ++i) ok &= t[i].y == epoch && t[i].w == epoch;
        return __all(ok) != 0;
      };
      auto h_take = [&](int slot, const uint4 (&t)[NLD]) {
        // two 4-byte LDS stores per word (one 8-byte store would need the
        // two values in adjacent registers, and the compiler would move them
        // there right after the load, waiting for it)
        lds_f32 *hs = lds(&s_hb[slot][0]);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int e = hb_pos(128 * i + 2 * lane);
          hs[e] = __uint_as_float(t[i].x);
          hs[e + 1] = __uint_as_float(t[i].z);
        }
      };
      auto release_routing = [&] {
        lds_release();
        if (lane == 0) *lds(&s_ready) = want;
        MOE_TRACE(2);
      };
      if (a.has_shared) {
#ifdef MOE_STACK_TRACE
        int nsh = 0;
#endif
        const bool done = poll_pipe<1, 8, 0, NLD>(
            [&](uint4 (&t)[NLD]) { h_issue(K, t); },
            [&](const uint4 (&t)[NLD]) {
#ifdef MOE_STACK_TRACE
              if (nsh++ == 0) MOE_TRACE(6);
#endif
              return h_ok(t);
            },
            [&](const uint4 (&t)[NLD]) { h_take(K, t); }, xspins, release_routing);
        if (!done && lane == 0) atomicOr(&a.ctrl->err, 2u);
        lds_release();
        if (lane == 0) *lds(&s_hready[K]) = want;
        MOE_TRACE(3);
      } else {
        release_routing();
      }
      uint32_t need = (1u << K) - 1u;  // routed slots not read yet
      while (need) {
        uint32_t pub = 0;
        for (int k = 0; k < K; ++k)
          if (((need >> k) & 1u) && *lds(&s_cnt[k]) >= (uint32_t)kGuWaves * want) pub |= 1u << k;
        pub = __builtin_amdgcn_readfirstlane(pub);
        if (pub) {
          // the two lowest such slots (two polls' words fit the registers)
          const int s0 = __builtin_ctz(pub);
          const uint32_t rest = pub & (pub - 1u);
          const int s1 = rest ? __builtin_ctz(rest) : -1;
          uint4 t0[NLD], t1[NLD];
          __asm__ volatile("" ::: "memory");
          h_issue(s0, t0);
          if (s1 >= 0) h_issue(s1, t1);
          auto settle = [&](int sl, uint4 (&t)[NLD]) {
            launder(t);
            if (h_ok(t)) {
              h_take(sl, t);
              lds_release();
              if (lane == 0) *lds(&s_hready[sl]) = want;
#ifdef MOE_STACK_TRACE
              if (lane == 0) s_tr[l * kTrEv + (sl < 3 ? 16 + sl : 4)] = __builtin_amdgcn_s_memrealtime();
#endif
              need &= ~(1u << sl);
            }
          };
          settle(s0, t0);
          if (s1 >= 0) settle(s1, t1);
        }
        if (need) {
          if (++xspins > kSpinMax) {
            if (lane == 0) atomicOr(&a.ctrl->err, 2u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    // every workgroup has passed the first layer's barrier, where it read the
    // epoch (this workgroup has read exchange words of all of them since)
    if (b == 0 && lane < kGroups)
      __hip_atomic_store(&a.fc->epoch[lane][0], s_epoch + (uint32_t)NL, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // =========================== down-row waves ===============================
    // The workgroup owns 16 y rows (a block, or every 256th row: the
    // MOE_STACK_ILV choice); waves 5, 6, 7 take 6, 6 and 4 of them, two rows
    // per wave-wide load (32 lanes each, 32 codes per lane), and compute
    // those rows of every slot: the shared
    // expert's as soon as its activations are in, then routed slot k's as
    // soon as slot k's are.  Each row's sum is formed as in k_layer1 (the
    // same lanes, products and reductions): y = shared + slot 0 + .. +
    // slot K-1, each slot's row already weighted by w_k.
    const int cw = wave - kGuWaves - 1;  // 0, 1, 2
    const int seg = lane % Gm::LPR;
    const size_t rbytes = (size_t)I * BITS / 8;
    const int groups = I / kGroup;
    static_assert(Gm::RPL == 2 && Gm::LPR == 32 && Gm::D_ROWS == 16, "rows per load and wave");
    auto o_dq = [&](int row) -> uint32_t {
      return (uint32_t)(a.off_dq + (int64_t)row * rbytes + seg * Gm::DWORDS * 4);
    };
    auto o_dsb = [&](int row) -> uint32_t {
      return (uint32_t)(a.off_dsb + ((int64_t)row * groups + seg * Gm::DCOLS / kGroup) * 4);
    };
    auto row_wave = [&](auto n_tag, int j0) {
      constexpr int N = decltype(n_tag)::value;  // wave-wide loads (row pairs) per slot
      int rows[N];
#pragma unroll
      for (int ld = 0; ld < N; ++ld) {
        const int j = j0 + 2 * ld + lane / Gm::LPR;  // the workgroup's j-th row
        rows[ld] = MOE_STACK_ILV ? j * kG + b : b * Gm::D_ROWS + j;
      }
      // residual mode: r of this lane's rows, kept across layers
      float rres[RES ? N : 1];
      if (RES) {
#pragma unroll
        for (int ld = 0; ld < N; ++ld) rres[ld] = a.resid[rows[ld]];
      }
      uint4 dq[NSL][N];
      uint32_t dsb[NSL][N];
      auto load_slot = [&](auto pol_tag, int slot, const uint8_t *bl) {
        constexpr int P = decltype(pol_tag)::value;
        const __amdgpu_buffer_rsrc_t rs = blob_rsrc(bl);
#pragma unroll
        for (int ld = 0; ld < N; ++ld) {
          if (Gm::DWORDS == 4) {
            dq[slot][ld] = bld16<P>(rs, o_dq(rows[ld]));
          } else {
            const uint2 v = bld8<P>(rs, o_dq(rows[ld]));
            dq[slot][ld] = make_uint4(v.x, v.y, 0u, 0u);
          }
          dsb[slot][ld] = bld4<P>(rs, o_dsb(rows[ld]));
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      for (int l = 0; l < NL; ++l) {
        const StackLayer Ly = uniform_layer(s_L[l]);
        if (RES) {
          gather_r(l, l == 0 ? 0u : s_epoch + (uint32_t)l);
          norm_x(l);
        }
        // the shared expert's rows (without one, slot K reads expert 0 and
        // is never used)
        if (MOE_STACK_RPF == 0 || l == 0)
          load_slot(std::integral_constant<int, kPolShared>{}, K,
                    a.has_shared ? Ly.shared : Ly.experts);
        if (l == 0 && tid == kEpochTid) s_epoch = epoch_done;
        lds_barrier();  // (A)
        const uint32_t want = (uint32_t)(l + 1);
        const uint32_t epoch = s_epoch + 1u + (uint32_t)l;
        if (cw == 2) {
          // this workgroup's logits, one copy per reader group (the sums of
          // the eight partials in wave order)
          if (lane < kCopies * rr) {
            const int rep = lane / rr, row = lane % rr, e = router_row(row);
            if (e < a.E) {
              float lg = 0.f;
#pragma unroll
              for (int w = 0; w < NW; ++w) lg += s_red[w][row];
              const uint64_t v = ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(lg);
              __hip_atomic_store(&a.tags[(size_t)rep * kMaxE + e], v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          MOE_TRACE(1);
        }
        wait_lds(&s_ready, want);
        if (cw == 2 && b == 0 && lane < K) {
          if (a.ids_out) a.ids_out[(size_t)l * K + lane] = s_ids[lane];
          if (a.w_out) a.w_out[(size_t)l * K + lane] = s_w[lane];
        }
        int eo[K];
        float wk[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          eo[k] = __builtin_amdgcn_readfirstlane(s_ids[k]);
          wk[k] = eo[k] >= 0 && eo[k] < a.E ? s_w[k] : 0.f;
        }
        float v[N];
#pragma unroll
        for (int ld = 0; ld < N; ++ld) v[ld] = 0.f;
        // the shared rows first: their activations come before any routed
        // slot's
        if (a.has_shared) {
          wait_lds(&s_hready[K], want);
          float acc[N];
#pragma unroll
          for (int ld = 0; ld < N; ++ld) acc[ld] = 0.f;
          down_rows<BITS, N, Gm::DWORDS, Gm::DCOLS>(dq[K], dsb[K], &s_hb[K][seg * Gm::DCOLS],
                                                     hb_key(seg),
                                                     1.f, acc);
#pragma unroll
          for (int ld = 0; ld < N; ++ld) v[ld] = lane_group_sum<Gm::LPR>(acc[ld], lane);
          if (cw == 0) MOE_TRACE(20);
        }
        if (MOE_STACK_RPF == 1 && l + 1 < NL && a.has_shared) {
          const StackLayer Ln = uniform_layer(s_L[l + 1]);
          load_slot(std::integral_constant<int, kPolShared>{}, K, Ln.shared);
        }
        // the routed rows' loads go after the gate/up waves' (the
        // activations, which every down row waits for, come from those
        // bytes), and only once this workgroup has published routed slot
        // MOE_STACK_RDELAY: until then the gate/up loads have the memory
        // pipeline to themselves
        if (MOE_STACK_RDELAY < 0) wait_lds(&s_gu_issued, (uint32_t)kGuWaves * want);
        else wait_lds(&s_cnt[MOE_STACK_RDELAY < K ? MOE_STACK_RDELAY : K - 1], (uint32_t)kGuWaves * want);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          // an invalid id reads expert 0 and contributes 0
          const bool ok = eo[k] >= 0 && eo[k] < a.E;
          load_slot(std::integral_constant<int, kPolRouted>{}, k,
                    Ly.experts + (size_t)(ok ? eo[k] : 0) * Ly.stride);
        }
        if (cw == 0) MOE_TRACE(19);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          wait_lds(&s_hready[k], want);
          float acc[N];
#pragma unroll
          for (int ld = 0; ld < N; ++ld) acc[ld] = 0.f;
          down_rows<BITS, N, Gm::DWORDS, Gm::DCOLS>(dq[k], dsb[k], &s_hb[k][seg * Gm::DCOLS],
                                                     hb_key(seg),
                                                     wk[k], acc);
#pragma unroll
          for (int ld = 0; ld < N; ++ld) v[ld] += lane_group_sum<Gm::LPR>(acc[ld], lane);
          if (cw == 0) MOE_TRACE(21 + k);
        }
#pragma unroll
        for (int ld = 0; ld < N; ++ld) {
          if (!RES) {
            if (seg == 0) a.y[(size_t)l * H + rows[ld]] = v[ld];
          } else {
            if (seg == 0 && a.y) a.y[(size_t)l * H + rows[ld]] = v[ld];
            rres[ld] = rres[ld] + v[ld];
            if (l + 1 < NL) {
              // r + y of this row for the next layer's norm, one copy per
              // reader group (lanes seg 0..7 of the row's lane group)
              if (seg < kCopies)
                __hip_atomic_store(&a.rtag[(size_t)seg * H + rows[ld]],
                                   ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(rres[ld]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (seg == 0) {
              a.resid[rows[ld]] = rres[ld];
            }
          }
        }
        if (RES && l + 1 < NL) {
          // the last of the three row waves to have stored its rows marks the
          // workgroup done, one copy per reader group
          uint32_t prev = 0;
          if (lane == 0)
            prev = __hip_atomic_fetch_add(&s_rstored, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
          prev = __builtin_amdgcn_readfirstlane(prev);
          if (prev + 1 == 3u * (uint32_t)(l + 1) && lane < kCopies)
            __hip_atomic_store(&a.rdone[(size_t)lane * kG + b], (uint64_t)epoch << 32,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (cw == 0) MOE_TRACE(7);
      }
    };
    if (cw < 2) row_wave(std::integral_constant<int, 3>{}, 6 * cw);
    else row_wave(std::integral_constant<int, 2>{}, 12);
  }
#ifdef MOE_STACK_TRACE
  __syncthreads();
  if (trace)
    for (int i = tid; i < NL * kTrEv; i += kNT) trace[(size_t)b * kMaxStackLayers * kTrEv + i] = s_tr[i];
#endif
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_stack_fused(const moe_dims &d, const moe_layer *layers, int n_layers,
                       const uint16_t *x, float *y, int32_t *ids_out, float *w_out, float *resid,
                       uint16_t *x_out, void *ws, void *stream) {
  if (n_layers < 1 || n_layers > kMaxStackLayers) return (int)hipErrorInvalidValue;
  const WsLayout W = ws_layout(d, 1);
  const BlobLayout B = blob_layout(d);
  uint8_t *base = static_cast<uint8_t *>(ws);
  StackArgs a;
  for (int l = 0; l < n_layers; ++l) {
    a.L[l].router = layers[l].router;
    a.L[l].experts = layers[l].experts;
    a.L[l].shared = layers[l].shared;
    a.L[l].stride = layers[l].expert_stride;
  }
  for (int l = n_layers; l < kMaxStackLayers; ++l) a.L[l] = a.L[0];
  a.n_layers = n_layers;
  a.x = x;
  a.y = y;
  a.ids_out = ids_out;
  a.w_out = w_out;
  a.resid = resid;
  a.x_out = x_out;
  a.ctrl = reinterpret_cast<Ctrl *>(base + W.ctrl);
  a.fc = reinterpret_cast<FCtrl *>(base + W.fctrl);
  a.tags = reinterpret_cast<uint64_t *>(base + W.logits_tag);
  a.htag = reinterpret_cast<uint64_t *>(base + W.h_tag);
  a.rtag = reinterpret_cast<uint64_t *>(base + W.r_tag);
  a.rdone = reinterpret_cast<uint64_t *>(base + W.r_done);
  a.E = d.n_experts;
  a.has_shared = d.has_shared;
  a.off_gq = (int64_t)B.off[MOE_SEC_GATE_Q];
  a.off_uq = (int64_t)B.off[MOE_SEC_UP_Q];
  a.off_dq = (int64_t)B.off[MOE_SEC_DOWN_Q];
  a.off_gsb = (int64_t)B.off[MOE_SEC_GATE_SB];
  a.off_usb = (int64_t)B.off[MOE_SEC_UP_SB];
  a.off_dsb = (int64_t)B.off[MOE_SEC_DOWN_SB];
  const int rr = (d.n_experts + kG - 1) / kG;
#define MOE_LAUNCH_ST(B, R, RS) \
  hipLaunchKernelGGL((k_stack<B, 4096, 1024, 4, R, RS>), dim3(kG), dim3(kNT), 0, S(stream), a)
#define MOE_LAUNCH_STR(B, RS)             \
  if (rr == 1) MOE_LAUNCH_ST(B, 1, RS);   \
  else if (rr == 2) MOE_LAUNCH_ST(B, 2, RS); \
  else MOE_LAUNCH_ST(B, 4, RS)
  if (d.bits == 4) {
    if (resid) { MOE_LAUNCH_STR(4, true); } else { MOE_LAUNCH_STR(4, false); }
  } else {
    if (resid) { MOE_LAUNCH_STR(2, true); } else { MOE_LAUNCH_STR(2, false); }
  }
#undef MOE_LAUNCH_STR
#undef MOE_LAUNCH_ST
  return (int)hipGetLastError();
}

}  // namespace moe
