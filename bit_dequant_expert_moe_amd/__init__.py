"""Thin ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the MoE layer runs in the HIP
kernels of libmoe.so.  Tensors are torch tensors on the current HIP device;
the stream is torch's current stream unless one is passed.  There is no CPU
fallback: importing fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB: another build of the library to load (the sanitizer test's)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_ALIGN", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP", -7: "MOE_ERR_DEVICE"}
SEC_GATE_Q, SEC_UP_Q, SEC_DOWN_Q, SEC_GATE_SB, SEC_UP_SB, SEC_DOWN_SB = range(6)
# bytes of the per-GPU workspace of moe_stack_decode_residual_noalloc
NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024
# code decoders of the kernel paths (moe_dequantize_as)
DEQ_SCALAR, DEQ_FP16_PAIR, DEQ_FP8_PAIR, DEQ_BF16_PAIR, DEQ_BF16_SLICE = range(5)

# Entry points that libmoe.so exports (one per declaration in include/moe.h).
EXPORTS = ("moe_abi_version", "moe_status_str", "moe_check_dims", "moe_expert_bytes",
           "moe_blob_layout", "moe_workspace_bytes", "moe_workspace_init", "moe_route",
           "moe_expert_forward", "moe_layer_decode", "moe_layer_decode_residual",
           "moe_dequantize", "moe_dequantize_as", "moe_get_device_error", "moe_tier_staging_bytes",
           "moe_tier_device_bytes", "moe_tier_workspace_bytes", "moe_tier_create",
           "moe_tier_decode", "moe_tier_plan", "moe_tier_stats", "moe_tier_destroy",
           "moe_stream_read_sink_words", "moe_stream_read", "moe_flush", "moe_stack_decode",
           "moe_stack_decode_residual", "moe_stack_decode_residual_noalloc", "moe_timing_set",
           "moe_timing_read")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (%d)" % (where, STATUS.get(status, "?"), status))
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "inter", "n_experts", "top_k", "group", "bits", "has_shared")]


class moe_layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("expert_stride", ctypes.c_int64), ("shared", ctypes.c_void_p)]


# per-stage timing: stage names in MOE_ST_* order
TIMING_STAGES = ("norm", "route", "bucket", "gateup", "down", "combine", "resid", "layer", "stack")


class moe_timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(TIMING_STAGES)),
                ("count", ctypes.c_int64 * len(TIMING_STAGES))]


class moe_tier_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("t_max", ctypes.c_int32),
                ("host_experts", ctypes.POINTER(ctypes.c_void_p)), ("host_stride", ctypes.c_int64),
                ("slots", ctypes.c_void_p), ("slot_stride", ctypes.c_int64),
                ("n_slots", ctypes.c_int32), ("copy_stream", ctypes.c_void_p),
                ("staging", ctypes.c_void_p), ("dev_scratch", ctypes.c_void_p)]


@dataclass(frozen=True)
class Dims:
    hidden: int = 4096
    inter: int = 1024
    n_experts: int = 512
    top_k: int = 4
    group: int = 64
    bits: int = 4
    has_shared: int = 1

    def c(self) -> moe_dims:
        return moe_dims(self.hidden, self.inter, self.n_experts, self.top_k, self.group,
                        self.bits, self.has_shared)


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp, lp = ctypes.POINTER(moe_dims), ctypes.POINTER(moe_layer)
        sig = {
            "moe_abi_version": (i32, []),
            "moe_status_str": (ctypes.c_char_p, [i32]),
            "moe_check_dims": (i32, [dp]),
            "moe_expert_bytes": (sz, [dp]),
            "moe_blob_layout": (i32, [dp, ctypes.POINTER(sz)]),
            "moe_workspace_bytes": (sz, [dp, i32]),
            "moe_workspace_init": (i32, [vp, sz, vp]),
            "moe_route": (i32, [dp, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_expert_forward": (i32, [dp, lp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_decode": (i32, [dp, lp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_decode_residual": (i32, [dp, lp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "moe_dequantize": (i32, [dp, vp, i32, vp, vp]),
            "moe_dequantize_as": (i32, [dp, vp, i32, i32, vp, vp]),
            "moe_get_device_error": (i32, [vp, vp, ctypes.POINTER(i32)]),
            "moe_tier_staging_bytes": (sz, [dp, i32]),
            "moe_tier_device_bytes": (sz, [dp, i32]),
            "moe_tier_workspace_bytes": (sz, [dp, i32, i32]),
            "moe_tier_create": (i32, [dp, ctypes.POINTER(moe_tier_config), ctypes.POINTER(vp)]),
            "moe_tier_decode": (i32, [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_tier_plan": (i32, [vp, i32, vp, i32, vp, vp]),
            "moe_tier_stats": (i32, [vp, ctypes.POINTER(ctypes.c_int64)]),
            "moe_tier_destroy": (None, [vp]),
            "moe_stream_read_sink_words": (sz, [sz]),
            "moe_stream_read": (i32, [vp, sz, vp, vp]),
            "moe_flush": (i32, [vp, sz, vp]),
            "moe_stack_decode": (i32, [dp, lp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "moe_stack_decode_residual": (i32, [dp, lp, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_stack_decode_residual_noalloc": (i32, [dp, lp, i32, vp, vp, vp, vp, vp, vp]),
            "moe_timing_set": (i32, [i32]),
            "moe_timing_read": (i32, [ctypes.POINTER(moe_timing), i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


# ---- host-only queries ---------------------------------------------------------

def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_check_dims(d: Dims) -> int:
    return int(lib().moe_check_dims(ctypes.byref(d.c())))


def moe_expert_bytes(d: Dims) -> int:
    return int(lib().moe_expert_bytes(ctypes.byref(d.c())))


def moe_blob_layout(d: Dims):
    out = (ctypes.c_size_t * 6)()
    _check(lib().moe_blob_layout(ctypes.byref(d.c()), out), "moe_blob_layout")
    return list(out)


def moe_workspace_bytes(d: Dims, T: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(d.c()), T))


# ---- device calls (enqueue on a stream) ---------------------------------------

def make_layer(router, experts, expert_stride: int, shared=None) -> moe_layer:
    return moe_layer(_ptr(router), _ptr(experts), int(expert_stride), _ptr(shared))


def moe_workspace_init(ws, ws_bytes: int, stream=None):
    _check(lib().moe_workspace_init(_ptr(ws), ws_bytes, _stream(stream)), "moe_workspace_init")


def alloc_workspace(d: Dims, T: int, device=None, stream=None):
    """Allocates (torch uint8, 256-byte aligned) and initialises a workspace."""
    import torch
    n = moe_workspace_bytes(d, T)
    if n == 0:
        raise MoeError(-2, "moe_workspace_bytes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device or "cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    moe_workspace_init(ws, n, stream)
    return ws


def moe_route(d: Dims, router, x, T: int, ids, w, logits=None, ws=None, ws_bytes=None,
              stream=None):
    rc = lib().moe_route(ctypes.byref(d.c()), _ptr(router), _ptr(x), T, _ptr(ids), _ptr(w),
                         _ptr(logits), _ptr(ws), ws_bytes if ws_bytes is not None else ws.numel(),
                         _stream(stream))
    _check(rc, "moe_route")


def moe_expert_forward(d: Dims, layer: moe_layer, x, T: int, ids, w, y, ws, ws_bytes=None,
                       stream=None):
    rc = lib().moe_expert_forward(ctypes.byref(d.c()), ctypes.byref(layer), _ptr(x), T,
                                  _ptr(ids), _ptr(w), _ptr(y), _ptr(ws),
                                  ws_bytes if ws_bytes is not None else ws.numel(),
                                  _stream(stream))
    _check(rc, "moe_expert_forward")


def moe_layer_decode(d: Dims, layer: moe_layer, x, T: int, y, ids=None, w=None, ws=None,
                     ws_bytes=None, stream=None):
    rc = lib().moe_layer_decode(ctypes.byref(d.c()), ctypes.byref(layer), _ptr(x), T, _ptr(y),
                                _ptr(ids), _ptr(w), _ptr(ws),
                                ws_bytes if ws_bytes is not None else ws.numel(),
                                _stream(stream))
    _check(rc, "moe_layer_decode")


def moe_layer_decode_residual(d: Dims, layer: moe_layer, resid, T: int, x_out=None, y=None,
                              ids=None, w=None, ws=None, ws_bytes=None, stream=None):
    rc = lib().moe_layer_decode_residual(ctypes.byref(d.c()), ctypes.byref(layer), _ptr(resid),
                                         T, _ptr(x_out), _ptr(y), _ptr(ids), _ptr(w), _ptr(ws),
                                         ws_bytes if ws_bytes is not None else ws.numel(),
                                         _stream(stream))
    _check(rc, "moe_layer_decode_residual")


def layer_array(layers) -> ctypes.Array:
    """A host array of moe_layer descriptors (keep it alive while in use)."""
    return (moe_layer * len(layers))(*layers)


def _layers(layers):
    return layers if isinstance(layers, ctypes.Array) else layer_array(layers)


def moe_stack_decode(d: Dims, layers, x, y, ids=None, w=None, ws=None, ws_bytes=None,
                     stream=None):
    """len(layers) consecutive layers of one token: x bf16 [L][H] -> y fp32
    [L][H] (ids/w [L][K] optional)."""
    arr = _layers(layers)
    rc = lib().moe_stack_decode(ctypes.byref(d.c()), arr, len(arr), _ptr(x), _ptr(y), _ptr(ids),
                                _ptr(w), _ptr(ws),
                                ws_bytes if ws_bytes is not None else ws.numel(), _stream(stream))
    _check(rc, "moe_stack_decode")


def moe_stack_decode_residual(d: Dims, layers, resid, x_out=None, y=None, ids=None, w=None,
                              ws=None, ws_bytes=None, stream=None):
    """len(layers) consecutive layers of one token on the residual stream
    resid fp32 [H] (updated in place)."""
    arr = _layers(layers)
    rc = lib().moe_stack_decode_residual(ctypes.byref(d.c()), arr, len(arr), _ptr(resid),
                                         _ptr(x_out), _ptr(y), _ptr(ids), _ptr(w), _ptr(ws),
                                         ws_bytes if ws_bytes is not None else ws.numel(),
                                         _stream(stream))
    _check(rc, "moe_stack_decode_residual")


def moe_stack_decode_residual_noalloc(d: Dims, layers, resid, x_out=None, y=None, ids=None,
                                      w=None, stream=None):
    """moe_stack_decode_residual on the library's own per-GPU workspace
    (allocates nothing; the first call on a GPU must not be captured)."""
    arr = _layers(layers)
    rc = lib().moe_stack_decode_residual_noalloc(ctypes.byref(d.c()), arr, len(arr), _ptr(resid),
                                                 _ptr(x_out), _ptr(y), _ptr(ids), _ptr(w),
                                                 _stream(stream))
    _check(rc, "moe_stack_decode_residual_noalloc")


def moe_dequantize(d: Dims, blob, which: int, out, stream=None):
    _check(lib().moe_dequantize(ctypes.byref(d.c()), _ptr(blob), which, _ptr(out),
                                _stream(stream)), "moe_dequantize")


def moe_dequantize_as(d: Dims, blob, which: int, decoder: int, out, stream=None):
    _check(lib().moe_dequantize_as(ctypes.byref(d.c()), _ptr(blob), which, decoder, _ptr(out),
                                   _stream(stream)), "moe_dequantize_as")


def moe_get_device_error(ws, stream=None) -> int:
    err = ctypes.c_int32(0)
    rc = lib().moe_get_device_error(_ptr(ws), _stream(stream), ctypes.byref(err))
    if rc not in (MOE_OK, -7):
        raise MoeError(rc, "moe_get_device_error")
    return int(err.value)


# ---- off-HBM expert tier ----------------------------------------------------------

class Tier:
    """moe_tier_* over caller-owned buffers.  host_ptrs: one host address per
    layer (pinned memory for asynchronous copies); slots, staging and
    dev_scratch are addresses (or tensors) the caller keeps alive."""

    def __init__(self, d: Dims, host_ptrs, host_stride: int, slots, slot_stride: int,
                 n_slots: int, staging, dev_scratch, t_max: int = 1, copy_stream=None):
        self.d = d
        self._hosts = (ctypes.c_void_p * len(host_ptrs))(*[int(p) for p in host_ptrs])
        cfg = moe_tier_config(len(host_ptrs), t_max, ctypes.cast(self._hosts,
                              ctypes.POINTER(ctypes.c_void_p)), int(host_stride), _ptr(slots),
                              int(slot_stride), n_slots, _ptr_stream(copy_stream), _ptr(staging),
                              _ptr(dev_scratch))
        self._cfg = cfg
        h = ctypes.c_void_p()
        _check(lib().moe_tier_create(ctypes.byref(d.c()), ctypes.byref(cfg), ctypes.byref(h)),
               "moe_tier_create")
        self.h = h
        self.n_slots = n_slots

    def plan(self, layer: int, ids, T: int):
        """Host-only slot plan for int32 host ids [T][K]; returns (slots, copies)."""
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        slots = np.empty(ids.size, dtype=np.int32)
        copies = np.empty(ids.size, dtype=np.int32)
        _check(lib().moe_tier_plan(self.h, layer, ids.ctypes.data, T, slots.ctypes.data,
                                   copies.ctypes.data), "moe_tier_plan")
        return slots, copies

    def decode(self, layer: int, router, shared, x, T: int, y, ids=None, w=None, ws=None,
               ws_bytes=None, stream=None):
        rc = lib().moe_tier_decode(self.h, layer, _ptr(router), _ptr(shared), _ptr(x), T, _ptr(y),
                                   _ptr(ids), _ptr(w), _ptr(ws),
                                   ws_bytes if ws_bytes is not None else ws.numel(),
                                   _stream(stream))
        _check(rc, "moe_tier_decode")

    def stats(self):
        out = (ctypes.c_int64 * 4)()
        _check(lib().moe_tier_stats(self.h, out), "moe_tier_stats")
        return dict(hits=out[0], misses=out[1], bytes=out[2], evictions=out[3])

    def close(self):
        if getattr(self, "h", None):
            lib().moe_tier_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr_stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def moe_tier_staging_bytes(d: Dims, t_max: int) -> int:
    return int(lib().moe_tier_staging_bytes(ctypes.byref(d.c()), t_max))


def moe_tier_device_bytes(d: Dims, t_max: int) -> int:
    return int(lib().moe_tier_device_bytes(ctypes.byref(d.c()), t_max))


def moe_tier_workspace_bytes(d: Dims, n_slots: int, T: int) -> int:
    return int(lib().moe_tier_workspace_bytes(ctypes.byref(d.c()), n_slots, T))


# ---- measurement helpers ---------------------------------------------------------

def moe_stream_read_sink_words(nbytes: int) -> int:
    return int(lib().moe_stream_read_sink_words(nbytes))


def moe_stream_read(src, nbytes: int, sink, stream=None):
    """One launch reading nbytes of device memory at src (a tensor or a
    device address); sink: int32/uint32 device tensor of
    moe_stream_read_sink_words(nbytes) words."""
    _check(lib().moe_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "moe_stream_read")


def moe_timing_set(on: bool):
    """Switches per-stage timing on or off."""
    _check(lib().moe_timing_set(1 if on else 0), "moe_timing_set")


def moe_timing_read(reset: bool = True) -> dict:
    """Per-stage totals since the last reset: {stage: (ms, count)} for the
    stages that ran (waits for the recorded events)."""
    t = moe_timing()
    _check(lib().moe_timing_read(ctypes.byref(t), 1 if reset else 0), "moe_timing_read")
    return {n: (t.ms[i], t.count[i]) for i, n in enumerate(TIMING_STAGES) if t.count[i]}


def moe_flush(dst, nbytes: int, stream=None):
    """One launch overwriting nbytes of device memory at dst."""
    _check(lib().moe_flush(_ptr(dst), nbytes, _stream(stream)), "moe_flush")
