// moe_host.cpp -- the C ABI of include/moe.h: argument validation, blob and
// workspace geometry, and dispatch to the kernel launchers.  Validation is
// pure host code and runs before anything is enqueued, so every error path
// is testable without a GPU.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_internal.h"

namespace moe {

static bool pow2_in(int v, int lo, int hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

static bool aligned(const void *p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

BlobLayout blob_layout(const moe_dims &d) {
  BlobLayout L;
  const size_t H = (size_t)d.hidden, I = (size_t)d.inter, b = (size_t)d.bits;
  const size_t g = (size_t)d.group;
  const size_t sizes[6] = {I * H * b / 8, I * H * b / 8, H * I * b / 8,
                           I * (H / g) * 4, I * (H / g) * 4, H * (I / g) * 4};
  size_t o = 0;
  for (int s = 0; s < 6; ++s) {
    L.off[s] = o;
    o = align_up(o + sizes[s], kAlign);
  }
  L.off[6] = o;
  return L;
}

WsLayout ws_layout(const moe_dims &d, int T) {
  WsLayout W;
  W.ctrl = kCtrlOff;
  W.fctrl = kFCtrlOff;
  W.logits_tag = kTagOff;
  W.h_tag = kHTagOff;
  W.p_tag = kPTagOff;
  W.r_tag = kRTagOff;
  W.r_done = kRDoneOff;
  size_t o = align_up(kHeaderBytes, kAlign);
  W.logits = o;
  o = align_up(o + (size_t)route_splits(d, T) * T * d.n_experts * 4, kAlign);
  W.ids = o;
  o = align_up(o + (size_t)T * d.top_k * 4, kAlign);
  W.w = o;
  o = align_up(o + (size_t)T * d.top_k * 4, kAlign);
  W.h = o;
  // indexed by pair code t (K + 1) + slot on every path
  o = align_up(o + (size_t)T * (d.top_k + 1) * d.inter * 4, kAlign);
  W.bk = W.xb = W.xs = W.hb = W.hs = W.yd = o;
  if (T >= 2) {
    const size_t P = (size_t)T * (d.top_k + 1);  // pair codes
    o = align_up(o + (size_t)grouped_bucket_words(d, T) * 4, kAlign);
    W.xb = o;
    o = align_up(o + (size_t)T * d.hidden * 2, kAlign);
    W.xs = o;
    o = align_up(o + (size_t)T * (d.hidden / kGroup) * 4, kAlign);
    W.hb = o;
    o = align_up(o + P * d.inter * 4, kAlign);
    W.hs = o;
    o = align_up(o + P * (d.inter / kGroup) * 4, kAlign);
    W.yd = o;
    o = align_up(o + P * d.hidden * 4, kAlign);
  }
  W.xn = o;
  o = align_up(o + (size_t)T * d.hidden * 2, kAlign);
  W.yr = o;
  o = align_up(o + (size_t)T * d.hidden * 4, kAlign);
  W.total = o;
  return W;
}

static moe_status check_dims(const moe_dims *d) {
  if (!d) return MOE_ERR_NULL;
  if (d->group != kGroup) return MOE_ERR_UNSUPPORTED;
  if (d->bits != 2 && d->bits != 4) return MOE_ERR_UNSUPPORTED;
  if (!pow2_in(d->hidden, 256, 16384) || !pow2_in(d->inter, 256, 16384)) return MOE_ERR_SHAPE;
  if (d->n_experts < 1 || d->n_experts > kMaxE) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > kMaxK || d->top_k > d->n_experts) return MOE_ERR_SHAPE;
  if (d->has_shared != 0 && d->has_shared != 1) return MOE_ERR_SHAPE;
  return MOE_OK;
}

static moe_status check_layer(const moe_dims *d, const moe_layer *L) {
  if (!L || !L->experts) return MOE_ERR_NULL;
  if (d->has_shared && !L->shared) return MOE_ERR_NULL;
  if (!d->has_shared && L->shared) return MOE_ERR_SHAPE;
  const size_t eb = blob_layout(*d).off[6];
  if (L->expert_stride < 0 || (size_t)L->expert_stride < eb) return MOE_ERR_SHAPE;
  if (L->expert_stride % (int64_t)kAlign != 0) return MOE_ERR_ALIGN;
  if (!aligned(L->experts, kAlign)) return MOE_ERR_ALIGN;
  if (L->shared && !aligned(L->shared, kAlign)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

static moe_status check_ws(const moe_dims *d, int T, const void *ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_NULL;
  if (!aligned(ws, kAlign)) return MOE_ERR_ALIGN;
  if (ws_bytes < ws_layout(*d, T).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// The single-token fused kernel is used when it covers the dims, for up to
// kFusedMaxT tokens (one launch each); setting MOE_DISABLE_FUSED=1 in the
// environment selects the three-kernel path for one token and the grouped
// path above (used to compare them).
static constexpr int kFusedMaxT = 3;
static bool use_fused(const moe_dims &d, int T) {
  static int disabled = -1;
  if (disabled < 0) {
    const char *e = getenv("MOE_DISABLE_FUSED");
    disabled = (e && e[0] == '1') ? 1 : 0;
  }
  return T <= kFusedMaxT && !disabled && fused_supported(d);
}

// Up to kFusedMaxT tokens run as one single-token launch each: there the
// grouped path's seven dependent launches cost more (one layer per call,
// measured: T = 2 60 us grouped against 41 us, T = 3 65 against 59; at T = 4
// the two are even).  Optional pointers advance with the token.
static int fused_tokens(const moe_dims &d, const moe_layer &L, const uint16_t *x, int T,
                        const int32_t *ids_in, const float *w_in, int32_t *ids_out,
                        float *w_out, float *y, float *resid, uint16_t *x_out, void *ws,
                        void *stream) {
  const size_t H = (size_t)d.hidden, K = (size_t)d.top_k;
  for (int t = 0; t < T; ++t) {
    timing::mark(MOE_ST_LAYER);
    const int rc = launch_layer_fused(
        d, L, x ? x + t * H : nullptr, ids_in ? ids_in + t * K : nullptr,
        w_in ? w_in + t * K : nullptr, ids_out ? ids_out + t * K : nullptr,
        w_out ? w_out + t * K : nullptr, y ? y + t * H : nullptr, resid ? resid + t * H : nullptr,
        x_out ? x_out + t * H : nullptr, ws, stream);
    if (rc != 0) return rc;
  }
  return 0;
}

// Stacks of layers run the multi-layer kernel where the single-token kernel
// covers the dims; MOE_DISABLE_STACK=1 runs one single-layer call per layer
// instead (used to compare the two).
static bool stack_disabled() {
  static int disabled = -1;
  if (disabled < 0) {
    const char *e = getenv("MOE_DISABLE_STACK");
    disabled = (e && e[0] == '1') ? 1 : 0;
  }
  return disabled == 1;
}

// Two or more tokens that the fused kernel does not take run the grouped path
// (pairs bucketed by expert, MFMA GEMMs); MOE_DISABLE_GROUPED=1 selects the
// per-token kernels instead.
static bool use_grouped(int T) {
  static int disabled = -1;
  if (disabled < 0) {
    const char *e = getenv("MOE_DISABLE_GROUPED");
    disabled = (e && e[0] == '1') ? 1 : 0;
  }
  return T >= 2 && !disabled;
}

static int expert_forward(const moe_dims &d, const moe_layer &L, const uint16_t *x, int T,
                          const int32_t *ids, const float *w, float *y, void *ws,
                          void *stream) {
  if (use_grouped(T)) return launch_expert_forward_grouped(d, L, x, T, ids, w, y, ws, stream);
  return launch_expert_forward(d, L, x, T, ids, w, y, ws, stream);
}

static moe_status check_T(int T) { return (T < 1 || T > kMaxT) ? MOE_ERR_SHAPE : MOE_OK; }

}  // namespace moe

using namespace moe;

#define MOE_TRY(expr)                \
  do {                               \
    moe_status s_ = (expr);          \
    if (s_ != MOE_OK) return s_;     \
  } while (0)

moe_status moe::check_stack_residual(const moe_dims *dims, const moe_layer *layers,
                                     int n_layers, const float *resid, const uint16_t *x_out,
                                     const float *y, const int32_t *ids, const float *w) {
  MOE_TRY(check_dims(dims));
  if (!layers || !resid) return MOE_ERR_NULL;
  if (n_layers < 1) return MOE_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    MOE_TRY(check_layer(dims, &layers[l]));
    if (!layers[l].router) return MOE_ERR_NULL;
    if (!aligned(layers[l].router, 16)) return MOE_ERR_ALIGN;
  }
  if (!aligned(resid, 16) || (x_out && !aligned(x_out, 16)) || (y && !aligned(y, 16)) ||
      (ids && !aligned(ids, 4)) || (w && !aligned(w, 4)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape or size";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_ALIGN: return "misaligned pointer or stride";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE: return "device reported invalid input";
  }
  return "unknown status";
}

moe_status moe_check_dims(const moe_dims *dims) { return check_dims(dims); }

size_t moe_expert_bytes(const moe_dims *dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return blob_layout(*dims).off[6];
}

moe_status moe_blob_layout(const moe_dims *dims, size_t out_offsets[6]) {
  MOE_TRY(check_dims(dims));
  if (!out_offsets) return MOE_ERR_NULL;
  BlobLayout L = blob_layout(*dims);
  for (int s = 0; s < 6; ++s) out_offsets[s] = L.off[s];
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_dims *dims, int32_t T) {
  if (check_dims(dims) != MOE_OK || check_T(T) != MOE_OK) return 0;
  return ws_layout(*dims, T).total;
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return MOE_ERR_NULL;
  if (!aligned(ws, kAlign)) return MOE_ERR_ALIGN;
  if (ws_bytes < kHeaderBytes) return MOE_ERR_WORKSPACE;
  return launch_ws_init(ws, ws_bytes, stream) == 0 ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_route(const moe_dims *dims, const uint16_t *router, const uint16_t *x,
                     int32_t T, int32_t *ids, float *w, float *logits, void *ws,
                     size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_T(T));
  if (!router || !x || !ids || !w) return MOE_ERR_NULL;
  if (!aligned(router, 16) || !aligned(x, 16) || !aligned(ids, 4) || !aligned(w, 4) ||
      (logits && !aligned(logits, 4)))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(dims, T, ws, ws_bytes));
  timing::Scope timed(stream);
  timing::mark(MOE_ST_ROUTE);
  return launch_route(*dims, router, x, T, ids, w, logits, ws, stream) == 0 ? MOE_OK
                                                                            : MOE_ERR_HIP;
}

moe_status moe_expert_forward(const moe_dims *dims, const moe_layer *layer, const uint16_t *x,
                              int32_t T, const int32_t *ids, const float *w, float *y,
                              void *ws, size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_T(T));
  MOE_TRY(check_layer(dims, layer));
  if (!x || !ids || !w || !y) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4) || !aligned(w, 4))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(dims, T, ws, ws_bytes));
  timing::Scope timed(stream);
  if (use_fused(*dims, T))
    return fused_tokens(*dims, *layer, x, T, ids, w, nullptr, nullptr, y, nullptr, nullptr, ws,
                        stream) == 0
               ? MOE_OK
               : MOE_ERR_HIP;
  return expert_forward(*dims, *layer, x, T, ids, w, y, ws, stream) == 0 ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_layer_decode(const moe_dims *dims, const moe_layer *layer, const uint16_t *x,
                            int32_t T, float *y, int32_t *ids, float *w, void *ws,
                            size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_T(T));
  MOE_TRY(check_layer(dims, layer));
  if (!x || !y) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || (ids && !aligned(ids, 4)) || (w && !aligned(w, 4)))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(dims, T, ws, ws_bytes));
  if (!layer->router) return MOE_ERR_NULL;
  if (!aligned(layer->router, 16)) return MOE_ERR_ALIGN;
  timing::Scope timed(stream);
  if (use_fused(*dims, T))
    return fused_tokens(*dims, *layer, x, T, nullptr, nullptr, ids, w, y, nullptr, nullptr, ws,
                        stream) == 0
               ? MOE_OK
               : MOE_ERR_HIP;
  const WsLayout W = ws_layout(*dims, T);
  uint8_t *base = static_cast<uint8_t *>(ws);
  int32_t *ids_d = ids ? ids : reinterpret_cast<int32_t *>(base + W.ids);
  float *w_d = w ? w : reinterpret_cast<float *>(base + W.w);
  timing::mark(MOE_ST_ROUTE);
  if (launch_route(*dims, layer->router, x, T, ids_d, w_d, nullptr, ws, stream) != 0)
    return MOE_ERR_HIP;
  if (expert_forward(*dims, *layer, x, T, ids_d, w_d, y, ws, stream) != 0) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_layer_decode_residual(const moe_dims *dims, const moe_layer *layer, float *resid,
                                     int32_t T, uint16_t *x_out, float *y, int32_t *ids,
                                     float *w, void *ws, size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_T(T));
  MOE_TRY(check_layer(dims, layer));
  if (!resid || !layer->router) return MOE_ERR_NULL;
  if (!aligned(resid, 16) || (x_out && !aligned(x_out, 16)) || (y && !aligned(y, 16)) ||
      (ids && !aligned(ids, 4)) || (w && !aligned(w, 4)) || !aligned(layer->router, 16))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(dims, T, ws, ws_bytes));
  timing::Scope timed(stream);
  if (use_fused(*dims, T))
    return fused_tokens(*dims, *layer, nullptr, T, nullptr, nullptr, ids, w, y, resid, x_out, ws,
                        stream) == 0
               ? MOE_OK
               : MOE_ERR_HIP;
  const WsLayout W = ws_layout(*dims, T);
  uint8_t *base = static_cast<uint8_t *>(ws);
  uint16_t *x_d = x_out ? x_out : reinterpret_cast<uint16_t *>(base + W.xn);
  float *y_d = y ? y : reinterpret_cast<float *>(base + W.yr);
  int32_t *ids_d = ids ? ids : reinterpret_cast<int32_t *>(base + W.ids);
  float *w_d = w ? w : reinterpret_cast<float *>(base + W.w);
  timing::mark(MOE_ST_NORM);
  if (launch_rmsnorm(*dims, resid, T, x_d, stream) != 0) return MOE_ERR_HIP;
  timing::mark(MOE_ST_ROUTE);
  if (launch_route(*dims, layer->router, x_d, T, ids_d, w_d, nullptr, ws, stream) != 0)
    return MOE_ERR_HIP;
  if (expert_forward(*dims, *layer, x_d, T, ids_d, w_d, y_d, ws, stream) != 0) return MOE_ERR_HIP;
  timing::mark(MOE_ST_RESID);
  if (launch_resid_add(*dims, resid, y_d, T, stream) != 0) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_stack_decode(const moe_dims *dims, const moe_layer *layers, int32_t n_layers,
                            const uint16_t *x, float *y, int32_t *ids, float *w, void *ws,
                            size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dims));
  if (!layers || !x || !y) return MOE_ERR_NULL;
  if (n_layers < 1) return MOE_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    MOE_TRY(check_layer(dims, &layers[l]));
    if (!layers[l].router) return MOE_ERR_NULL;
    if (!aligned(layers[l].router, 16)) return MOE_ERR_ALIGN;
  }
  if (!aligned(x, 16) || !aligned(y, 16) || (ids && !aligned(ids, 4)) || (w && !aligned(w, 4)))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(dims, 1, ws, ws_bytes));
  timing::Scope timed(stream);
  const size_t H = (size_t)dims->hidden, K = (size_t)dims->top_k;
  if (use_fused(*dims, 1) && !stack_disabled()) {
    for (int l0 = 0; l0 < n_layers; l0 += kMaxStackLayers) {
      const int n = n_layers - l0 < kMaxStackLayers ? n_layers - l0 : kMaxStackLayers;
      timing::mark(MOE_ST_STACK);
      if (launch_stack_fused(*dims, layers + l0, n, x + l0 * H, y + l0 * H,
                             ids ? ids + l0 * K : nullptr, w ? w + l0 * K : nullptr, nullptr,
                             nullptr, ws, stream) != 0)
        return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const moe_status st = moe_layer_decode(dims, &layers[l], x + l * H, 1, y + l * H,
                                           ids ? ids + l * K : nullptr, w ? w + l * K : nullptr,
                                           ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_stack_decode_residual(const moe_dims *dims, const moe_layer *layers,
                                     int32_t n_layers, float *resid, uint16_t *x_out, float *y,
                                     int32_t *ids, float *w, void *ws, size_t ws_bytes,
                                     void *stream) {
  MOE_TRY(check_stack_residual(dims, layers, n_layers, resid, x_out, y, ids, w));
  MOE_TRY(check_ws(dims, 1, ws, ws_bytes));
  timing::Scope timed(stream);
  const size_t H = (size_t)dims->hidden, K = (size_t)dims->top_k;
  if (use_fused(*dims, 1) && !stack_disabled()) {
    for (int l0 = 0; l0 < n_layers; l0 += kMaxStackLayers) {
      const int n = n_layers - l0 < kMaxStackLayers ? n_layers - l0 : kMaxStackLayers;
      timing::mark(MOE_ST_STACK);
      if (launch_stack_fused(*dims, layers + l0, n, nullptr, y ? y + l0 * H : nullptr,
                             ids ? ids + l0 * K : nullptr, w ? w + l0 * K : nullptr, resid,
                             x_out ? x_out + l0 * H : nullptr, ws, stream) != 0)
        return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const moe_status st = moe_layer_decode_residual(
        dims, &layers[l], resid, 1, x_out ? x_out + l * H : nullptr, y ? y + l * H : nullptr,
        ids ? ids + l * K : nullptr, w ? w + l * K : nullptr, ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_dequantize_as(const moe_dims *dims, const uint8_t *blob, int32_t which,
                             int32_t decoder, float *out, void *stream) {
  MOE_TRY(check_dims(dims));
  if (!blob || !out) return MOE_ERR_NULL;
  if (which < 0 || which > 2) return MOE_ERR_SHAPE;
  if (decoder < MOE_DEQ_SCALAR || decoder > MOE_DEQ_BF16_SLICE) return MOE_ERR_SHAPE;
  if (!aligned(blob, kAlign) || !aligned(out, 16)) return MOE_ERR_ALIGN;
  return launch_dequantize_as(*dims, blob, which, decoder, out, stream) == 0 ? MOE_OK
                                                                              : MOE_ERR_HIP;
}

moe_status moe_dequantize(const moe_dims *dims, const uint8_t *blob, int32_t which, float *out,
                          void *stream) {
  // the decoders of the single-token kernel: fp16 pairs for gate and up,
  // the fp8 pair convert for down
  return moe_dequantize_as(dims, blob, which, which == 2 ? MOE_DEQ_FP8_PAIR : MOE_DEQ_FP16_PAIR,
                           out, stream);
}

size_t moe_stream_read_sink_words(size_t bytes) {
  return (size_t)stream_read_blocks(bytes);
}

moe_status moe_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink) return MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return MOE_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGN;
  return launch_stream_read(src, bytes, sink, stream) == 0 ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_timing_set(int32_t on) {
  timing::set(on != 0);
  return MOE_OK;
}

moe_status moe_timing_read(moe_timing *out, int32_t reset) {
  if (!out) return MOE_ERR_NULL;
  return timing::read(out->ms, out->count, reset != 0) == 0 ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_flush(void *dst, size_t bytes, void *stream) {
  if (!dst) return MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return MOE_ERR_SHAPE;
  if (!aligned(dst, 16)) return MOE_ERR_ALIGN;
  return launch_flush(dst, bytes, stream) == 0 ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_get_device_error(void *ws, void *stream, int32_t *err) {
  if (!ws || !err) return MOE_ERR_NULL;
  if (!aligned(ws, kAlign)) return MOE_ERR_ALIGN;
  if (read_device_error(ws, stream, err) != 0) return MOE_ERR_HIP;
  return *err ? MOE_ERR_DEVICE : MOE_OK;
}

}  // extern "C"
