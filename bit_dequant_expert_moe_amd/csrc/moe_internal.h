// moe_internal.h -- shared declarations between the host ABI (moe_host.cpp)
// and the kernels (moe_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kGroup = 64;
constexpr int kMaxT = 4096;  // tokens per call (a prefill chunk)
constexpr int kMaxK = 8;
constexpr int kMaxE = 1024;
constexpr size_t kAlign = 256;
constexpr int kMaxRouteSplits = 8;

inline size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Byte offsets of the six blob sections plus the total (offsets[6]).
struct BlobLayout {
  size_t off[7];
};
BlobLayout blob_layout(const moe_dims &d);

// Workspace map (byte offsets from the workspace base).  The first
// kHeaderBytes hold control words and are zeroed by moe_workspace_init:
//   ctrl       : Ctrl (256 bytes)
//   fctrl      : FCtrl (epoch of the fused single-token kernel)
//   logits_tag : uint64 [kGroups][kMaxE]  (fp32 logit bits | epoch << 32)
//   h_tag      : uint64 [kGroups][5][1024] (fp32 h bits | epoch << 32)
//   p_tag      : uint64 [4][4096]  routed down sums per slot and output row
//                (fp32 bits | epoch << 32)
//   r_tag      : uint64 [kGroups][4096] r + y per output row (multi-layer
//                kernel, residual mode)
//   r_done     : uint64 [kGroups][256] per workgroup: its rows of r_tag are
//                stored (epoch in the high half)
// then, not initialised:
//   logits     : fp32 [S][T][E] partial router sums (S <= kMaxRouteSplits)
//   ids        : int32 [T][K]
//   w          : fp32 [T][K]
//   h          : fp32 [T][K+1][I]   activations silu(g)*u per slot
//   batched path (T >= 2) only:
//   bk         : int32 buckets (expert, offsets, pair codes, work items)
//   xb, xs     : x as matrix-core B operand [T][H/8] x 16 B, group sums [T][H/64]
//   hb, hs     : h as B operand [T][K+1][I/8] x 32 B (bf16 hi, lo), sums [T][K+1][I/64]
//   yd         : fp32 [T][K+1][H]   per-slot down projections
//   residual entry point, unfused path only:
//   xn         : bf16 [T][H]   normalised x (when the caller passes no x_out)
//   yr         : fp32 [T][H]   layer output (when the caller passes no y)
struct Ctrl {
  uint32_t reserved;       // unused
  uint32_t err;            // sticky device error flags
  uint32_t pad[62];
};
static_assert(sizeof(Ctrl) == 256, "control block is 256 bytes");

constexpr int kGroups = 8;  // workgroup groups by blockIdx % 8 (one per XCD)
// Synchronisation state of the fused single-token kernel.  Every datum that
// all workgroups read is stored once per reader group (kGroups copies), so
// each cache line has ~32 coherent readers instead of 256 (coherent reads of
// one line from every CU serialise at its memory channel).  Data words carry
// the epoch of the call that wrote them in their upper 32 bits, so a reader
// detects completion from the data itself.
struct FCtrl {
  // calls completed on this workspace, one copy per reader group, each on a
  // cache line of its own
  uint32_t epoch[kGroups][32];
};
static_assert(sizeof(FCtrl) == 1024, "epoch copies are 128 bytes apart");
constexpr int kFusedI = 1024;     // intermediate size the fused kernel covers
constexpr int kFusedSlots = 5;    // top-4 + shared
constexpr int kFusedH = 4096;     // hidden size the fused kernel covers

constexpr size_t kCtrlOff = 0;
constexpr size_t kFCtrlOff = 256;
// tagged logits: uint64 [kGroups][kMaxE]
constexpr size_t kTagOff = kFCtrlOff + sizeof(FCtrl);
// tagged activations: uint64 [kGroups][kFusedSlots][kFusedI]
constexpr size_t kHTagOff = kTagOff + (size_t)kGroups * kMaxE * 8;
// tagged routed down sums: uint64 [kFusedSlots - 1][kFusedH]
constexpr size_t kPTagOff = kHTagOff + (size_t)kGroups * kFusedSlots * kFusedI * 8;
// tagged residual rows r + y of the multi-layer kernel: uint64 [kGroups][kFusedH]
constexpr size_t kRTagOff = kPTagOff + (size_t)(kFusedSlots - 1) * kFusedH * 8;
// one tagged word per workgroup once its r + y rows are stored: uint64 [kGroups][256]
constexpr size_t kRDoneOff = kRTagOff + (size_t)kGroups * kFusedH * 8;
constexpr size_t kHeaderBytes = kRDoneOff + (size_t)kGroups * 256 * 8;
constexpr int kMaxStackLayers = 64;  // layers per launch of the multi-layer kernel

struct WsLayout {
  size_t ctrl, fctrl, logits_tag, h_tag, p_tag, r_tag, r_done, logits, ids, w, h, bk, xb, xs, hb, hs, yd,
      xn, yr, total;
};
WsLayout ws_layout(const moe_dims &d, int T);

// Geometry of one matrix row in 16-byte segments as the GEMV kernels see it.
struct RowGeo {
  int seg_per_row;  // row bytes / 16
  int lpr;          // lanes of a wave that share one row (<= 64)
  int rpl;          // rows covered by one wave-wide load (64 / lpr)
  int nseg;         // segments per lane per row (seg_per_row / lpr)
};
inline RowGeo row_geo(int cols, int bits) {
  RowGeo g;
  g.seg_per_row = cols * bits / 128;
  g.lpr = g.seg_per_row < 64 ? g.seg_per_row : 64;
  g.rpl = 64 / g.lpr;
  g.nseg = g.seg_per_row / g.lpr;
  return g;
}

// From this many tokens the router runs in 64-token x 64-expert tiles with
// both operands staged in LDS (k_router_tiled); below, in 16 x 16 tiles that
// read their operands straight from memory (k_router).
constexpr int kRouteTiledT = 512;
inline bool route_tiled(int T) { return T >= kRouteTiledT; }

// Column splits of the router for T tokens: the blocks (16 x 16 or 64 x 64
// tiles) are split along the hidden dimension until about 256 blocks stream
// the router (16 x 16: each wave keeps whole 32-column steps; 64 x 64: each
// split whole 64-column steps).
inline int route_splits(const moe_dims &d, int T) {
  const int tile = route_tiled(T) ? 64 : 16;
  const int per_split = route_tiled(T) ? 64 : 128;
  const int blocks = ((d.n_experts + tile - 1) / tile) * ((T + tile - 1) / tile);
  int s = 1;
  while (s < kMaxRouteSplits && blocks * s < 256 && d.hidden % (per_split * 2 * s) == 0) s *= 2;
  return s;
}

// Per-stage timing (moe_timing.cpp): an entry point opens a call on its
// stream, marks the start of each stage (MOE_ST_*) and closes the call; all
// no-ops while timing is off or the stream is being captured.  Calls nest:
// only the outermost records.
namespace timing {
bool on();
void set(bool enable);
void begin(void *stream);
void mark(int stage);
void end();
// waits for the closed calls' events and adds them to the totals; copies the
// totals out (and zeroes them with reset); -1 if an event call failed
int read(double *ms, int64_t *count, bool reset);
// opens a call for the lifetime of the object
struct Scope {
  explicit Scope(void *stream) { begin(stream); }
  ~Scope() { end(); }
  Scope(const Scope &) = delete;
  Scope &operator=(const Scope &) = delete;
};
}  // namespace timing

// Kernel launchers (moe_kernels.hip).  Each returns hipSuccess (0) or the
// HIP error of the launch.
int launch_ws_init(void *ws, size_t bytes, void *stream);
// Argument checks of moe_stack_decode_residual other than the workspace's.
moe_status check_stack_residual(const moe_dims *dims, const moe_layer *layers, int n_layers,
                                const float *resid, const uint16_t *x_out, const float *y,
                                const int32_t *ids, const float *w);
int launch_route(const moe_dims &d, const uint16_t *router, const uint16_t *x, int T,
                 int32_t *ids, float *w, float *logits, void *ws, void *stream);
int launch_expert_forward(const moe_dims &d, const moe_layer &L, const uint16_t *x, int T,
                          const int32_t *ids, const float *w, float *y, void *ws,
                          void *stream);
bool fused_supported(const moe_dims &d);
// With resid != null the kernel runs in residual mode: x is formed from resid
// (written to x_out if given), resid += y in place, y is optional.
int launch_layer_fused(const moe_dims &d, const moe_layer &L, const uint16_t *x,
                       const int32_t *ids_in, const float *w_in, int32_t *ids_out,
                       float *w_out, float *y, float *resid, uint16_t *x_out, void *ws,
                       void *stream);
// n_layers (<= kMaxStackLayers) consecutive layers of one token in one launch
// (moe_stack.hip); resid != null selects residual mode (x from resid, x_out
// optional, y optional), else x [n_layers][H] and y [n_layers][H].
int launch_stack_fused(const moe_dims &d, const moe_layer *layers, int n_layers,
                       const uint16_t *x, float *y, int32_t *ids_out, float *w_out, float *resid,
                       uint16_t *x_out, void *ws, void *stream);
// Residual stream steps of the unfused path.
int launch_rmsnorm(const moe_dims &d, const float *r, int T, uint16_t *x, void *stream);
int launch_resid_add(const moe_dims &d, float *r, const float *y, int T, void *stream);
// One matrix of a blob as fp32 through the unpack of `decoder` (MOE_DEQ_*).
int launch_dequantize_as(const moe_dims &d, const uint8_t *blob, int which, int decoder,
                         float *out, void *stream);
namespace dev {
struct DequantArgs;
}
int launch_dequant_fp8(const dev::DequantArgs &a, int blocks, void *stream);     // moe_fused.hip
int launch_dequant_slices(const dev::DequantArgs &a, int blocks, void *stream);  // moe_grouped.hip
// Batched path (moe_grouped.hip): pairs grouped by expert, MFMA GEMMs.
int grouped_max_buckets(const moe_dims &d, int T);
int grouped_bucket_words(const moe_dims &d, int T);  // int32 words of the bucket area
int launch_expert_forward_grouped(const moe_dims &d, const moe_layer &L, const uint16_t *x,
                                  int T, const int32_t *ids, const float *w, float *y, void *ws,
                                  void *stream);
int read_device_error(void *ws, void *stream, int32_t *err);
// Measurement kernels (moe_probe.hip).
int stream_read_blocks(size_t bytes);
int launch_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
int launch_flush(void *dst, size_t bytes, void *stream);

}  // namespace moe
