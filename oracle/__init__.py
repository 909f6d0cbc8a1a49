"""Float64 CPU oracle of one MoE layer (test infrastructure only).

Only the tests, the package's ``smoke()`` check and the benchmark's CPU
baseline import this module.  It wraps ``oracle.c`` (plain sequential double
loops) through ctypes; it shares no code with the HIP library.

What is computed, per the Flash-MoE pages ("Flash-MoE: Running a 397B
Parameter Model on a Laptop", hysenlabs.com, section "How the SSD expert
streaming pipeline works"; "Flash-MoE: Running a 400 Billion Parameter Model
on a MacBook", mattcullerton.com, section "The Architecture"): router logits,
softmax, top-K, renormalised weights, the dequantised SwiGLU expert MLP of the
selected experts plus the shared expert, and the weighted combine.  The
readings taken where the pages are silent are listed in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("H", "I", "E", "K", "bits", "group", "has_shared")]


@dataclass(frozen=True)
class Dims:
    """Layer shape as the oracle sees it."""
    H: int
    I: int
    E: int
    K: int
    bits: int = 4
    group: int = 64
    has_shared: int = 1

    def c(self) -> _Dims:
        return _Dims(self.H, self.I, self.E, self.K, self.bits, self.group, self.has_shared)


def build(force: bool = True, out: str = None, extra=None) -> str:
    """Compiles oracle.c with gcc (no fast-math, no FMA contraction) into
    liboracle.so, or into `out` with the extra flags `extra` (e.g. a
    sanitizer build)."""
    dst = out or _LIB
    if force or not os.path.exists(dst) or os.path.getmtime(dst) < os.path.getmtime(_SRC):
        tmp = dst + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off",
                               "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", *(extra or []),
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, dst)
    return dst


_lib = None


def lib():
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIB: a prebuilt oracle library to load instead (the
        # sanitizer test builds one)
        path = os.environ.get("MOE_ORACLE_LIB") or build(force=False)
        L = ctypes.CDLL(path)
        dp = ctypes.POINTER(_Dims)
        L.or_set_threads.restype = None
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_get_threads.restype = ctypes.c_int
        L.or_get_threads.argtypes = []
        L.or_bf16.restype = ctypes.c_double
        L.or_bf16.argtypes = [ctypes.c_uint16]
        L.or_section_offset.restype = ctypes.c_int64
        L.or_section_offset.argtypes = [dp, ctypes.c_int]
        L.or_blob_bytes.restype = ctypes.c_int64
        L.or_blob_bytes.argtypes = [dp]
        L.or_code.restype = ctypes.c_int32
        L.or_code.argtypes = [dp, _u8p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        L.or_scale_bias.restype = None
        L.or_scale_bias.argtypes = [dp, _u8p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    _f64p, _f64p]
        L.or_dequant.restype = ctypes.c_double
        L.or_dequant.argtypes = [dp, _u8p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        L.or_dequant_f32.restype = ctypes.c_float
        L.or_dequant_f32.argtypes = [dp, _u8p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        L.or_dequant_matrix.restype = None
        L.or_dequant_matrix.argtypes = [dp, _u8p, ctypes.c_int, _f64p]
        L.or_dequant_matrix_f32.restype = None
        L.or_dequant_matrix_f32.argtypes = [dp, _u8p, ctypes.c_int, _f32p]
        L.or_router_logits.restype = None
        L.or_router_logits.argtypes = [dp, _u16p, _u16p, _f64p]
        L.or_route_token.restype = None
        L.or_route_token.argtypes = [dp, _f64p, _i32p, _f64p, _f64p]
        L.or_route.restype = None
        L.or_route.argtypes = [dp, _u16p, _u16p, ctypes.c_int32, _i32p, _f64p, _f64p, _f64p]
        L.or_silu.restype = ctypes.c_double
        L.or_silu.argtypes = [ctypes.c_double]
        L.or_expert.restype = None
        L.or_expert.argtypes = [dp, _u8p, _f64p, _f64p, _f64p]
        L.or_layer.restype = None
        L.or_layer.argtypes = [dp, _u16p, ctypes.POINTER(_u8p), _u8p, _u16p, ctypes.c_int32,
                               _f64p, _i32p, _f64p, _f64p, _f64p]
        L.or_expert_forward.restype = None
        L.or_expert_forward.argtypes = [dp, ctypes.POINTER(_u8p), _u8p, _u16p, ctypes.c_int32,
                                        _i32p, _f64p, _f64p]
        L.or_f64_to_bf16.restype = ctypes.c_uint16
        L.or_f64_to_bf16.argtypes = [ctypes.c_double]
        L.or_rmsnorm_bf16.restype = None
        L.or_rmsnorm_bf16.argtypes = [ctypes.c_int64, _f32p, ctypes.c_double, _u16p]
        L.or_residual_layer.restype = None
        L.or_residual_layer.argtypes = [dp, _u16p, ctypes.POINTER(_u8p), _u8p, _f32p,
                                        ctypes.c_int32, _f64p, _u16p, _f64p, _i32p, _f64p,
                                        _f64p, _f64p]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads for independent output rows (1: sequential).  Results are the
    same for every thread count."""
    lib().or_set_threads(int(n))


def get_threads() -> int:
    return int(lib().or_get_threads())


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def section_offset(d: Dims, sec: int) -> int:
    return int(lib().or_section_offset(ctypes.byref(d.c()), sec))


def blob_bytes(d: Dims) -> int:
    return int(lib().or_blob_bytes(ctypes.byref(d.c())))


def code(d: Dims, blob: np.ndarray, which: int, r: int, c: int) -> int:
    blob = _c(blob, np.uint8)
    return int(lib().or_code(ctypes.byref(d.c()), _p(blob, _u8p), which, r, c))


def scale_bias(d: Dims, blob: np.ndarray, which: int, r: int, c: int):
    blob = _c(blob, np.uint8)
    s, z = ctypes.c_double(), ctypes.c_double()
    lib().or_scale_bias(ctypes.byref(d.c()), _p(blob, _u8p), which, r, c,
                        ctypes.byref(s), ctypes.byref(z))
    return s.value, z.value


def dequant(d: Dims, blob: np.ndarray, which: int, r: int, c: int) -> float:
    blob = _c(blob, np.uint8)
    return float(lib().or_dequant(ctypes.byref(d.c()), _p(blob, _u8p), which, r, c))


def _shape(d: Dims, which: int):
    return (d.H, d.I) if which == 2 else (d.I, d.H)


def dequant_matrix(d: Dims, blob: np.ndarray, which: int) -> np.ndarray:
    """Exact dequantised matrix `which` (0 gate, 1 up, 2 down) in float64."""
    blob = _c(blob, np.uint8)
    out = np.empty(_shape(d, which), dtype=np.float64)
    lib().or_dequant_matrix(ctypes.byref(d.c()), _p(blob, _u8p), which, _p(out, _f64p))
    return out


def dequant_matrix_f32(d: Dims, blob: np.ndarray, which: int) -> np.ndarray:
    """The same, each element rounded once to fp32."""
    blob = _c(blob, np.uint8)
    out = np.empty(_shape(d, which), dtype=np.float32)
    lib().or_dequant_matrix_f32(ctypes.byref(d.c()), _p(blob, _u8p), which, _p(out, _f32p))
    return out


def router_logits(d: Dims, router: np.ndarray, x: np.ndarray) -> np.ndarray:
    router, x = _c(router, np.uint16), _c(x, np.uint16)
    out = np.empty(d.E, dtype=np.float64)
    lib().or_router_logits(ctypes.byref(d.c()), _p(router, _u16p), _p(x, _u16p), _p(out, _f64p))
    return out


def route_logits(d: Dims, logits: np.ndarray):
    """Softmax -> top-K -> renormalise for one token's logits (float64 [E])."""
    logits = _c(logits, np.float64)
    ids = np.empty(d.K, dtype=np.int32)
    w = np.empty(d.K, dtype=np.float64)
    gap = ctypes.c_double()
    lib().or_route_token(ctypes.byref(d.c()), _p(logits, _f64p), _p(ids, _i32p), _p(w, _f64p),
                         ctypes.byref(gap))
    return ids, w, gap.value


def route(d: Dims, router: np.ndarray, x: np.ndarray):
    """Routing of T tokens: returns ids [T][K], w [T][K], logits [T][E], gap [T]."""
    router = _c(router, np.uint16)
    x = _c(x, np.uint16).reshape(-1, d.H)
    T = x.shape[0]
    ids = np.empty((T, d.K), dtype=np.int32)
    w = np.empty((T, d.K), dtype=np.float64)
    logits = np.empty((T, d.E), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    lib().or_route(ctypes.byref(d.c()), _p(router, _u16p), _p(x, _u16p), T, _p(ids, _i32p),
                   _p(w, _f64p), _p(logits, _f64p), _p(gap, _f64p))
    return ids, w, logits, gap


def silu(v: float) -> float:
    return float(lib().or_silu(v))


def expert(d: Dims, blob: np.ndarray, x: np.ndarray, want_h: bool = False):
    """One expert MLP on one token; x is float64 [H] (or bf16 bits uint16)."""
    blob = _c(blob, np.uint8)
    x = np.asarray(x)
    xd = bf16_to_f64(x) if x.dtype == np.uint16 else _c(x, np.float64)
    y = np.empty(d.H, dtype=np.float64)
    h = np.empty(d.I, dtype=np.float64)
    lib().or_expert(ctypes.byref(d.c()), _p(blob, _u8p), _p(xd, _f64p), _p(y, _f64p),
                    _p(h, _f64p))
    return (y, h) if want_h else y


def _blob_table(d: Dims, blobs):
    """blobs: dict expert -> uint8 array (host).  Returns (ctypes array, keepalive)."""
    keep = []
    arr = (_u8p * d.E)()
    for e, b in blobs.items():
        b = _c(b, np.uint8)
        keep.append(b)
        arr[e] = _p(b, _u8p)
    return arr, keep


def layer(d: Dims, router: np.ndarray, blobs, shared, x: np.ndarray):
    """Full layer for T tokens.  blobs: mapping expert -> host blob (uint8),
    or a callable expert -> blob; only the selected experts are fetched.
    Returns y [T][H] float64, ids, w, logits, gap."""
    router = _c(router, np.uint16)
    x = _c(x, np.uint16).reshape(-1, d.H)
    T = x.shape[0]
    ids0, _, _, _ = route(d, router, x)
    if callable(blobs):
        blobs = {int(e): blobs(int(e)) for e in np.unique(ids0)}
    arr, keep = _blob_table(d, blobs)
    sh = _c(shared, np.uint8) if d.has_shared else None
    y = np.empty((T, d.H), dtype=np.float64)
    ids = np.empty((T, d.K), dtype=np.int32)
    w = np.empty((T, d.K), dtype=np.float64)
    logits = np.empty((T, d.E), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    lib().or_layer(ctypes.byref(d.c()), _p(router, _u16p), arr,
                   _p(sh, _u8p) if sh is not None else None, _p(x, _u16p), T, _p(y, _f64p),
                   _p(ids, _i32p), _p(w, _f64p), _p(logits, _f64p), _p(gap, _f64p))
    del keep
    return y, ids, w, logits, gap


def expert_forward(d: Dims, blobs, shared, x: np.ndarray, ids: np.ndarray, w: np.ndarray):
    """Expert forward + combine with given routing (ids [T][K], w [T][K])."""
    x = _c(x, np.uint16).reshape(-1, d.H)
    T = x.shape[0]
    ids = _c(ids, np.int32).reshape(T, d.K)
    w = _c(w, np.float64).reshape(T, d.K)
    if callable(blobs):
        blobs = {int(e): blobs(int(e)) for e in np.unique(ids) if 0 <= e < d.E}
    arr, keep = _blob_table(d, blobs)
    sh = _c(shared, np.uint8) if d.has_shared else None
    y = np.empty((T, d.H), dtype=np.float64)
    lib().or_expert_forward(ctypes.byref(d.c()), arr, _p(sh, _u8p) if sh is not None else None,
                            _p(x, _u16p), T, _p(ids, _i32p), _p(w, _f64p), _p(y, _f64p))
    del keep
    return y


RMS_EPS = 1e-6


def f64_to_bf16(v: float) -> int:
    """Nearest bf16 bit pattern of a double (via float, ties to even)."""
    return int(lib().or_f64_to_bf16(float(v)))


def rmsnorm_bf16(r: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """x = bf16(r / sqrt(mean(r^2) + eps)) per row of an fp32 [T][n] array."""
    r = _c(r, np.float32)
    r2 = r.reshape(-1, r.shape[-1])
    x = np.empty(r2.shape, dtype=np.uint16)
    for t in range(r2.shape[0]):
        lib().or_rmsnorm_bf16(r2.shape[1], _p(r2[t], _f32p), eps, _p(x[t], _u16p))
    return x.reshape(r.shape)


def residual_layer(d: Dims, router: np.ndarray, blobs, shared, r: np.ndarray):
    """One MoE layer on the fp32 residual stream r [T][H]: x = rmsnorm(r)
    (bf16), y = layer(x), r_out = r + y.  blobs as in layer().  Returns
    r_out (float64), x (bf16 bits), y, ids, w, logits, gap."""
    router = _c(router, np.uint16)
    r = _c(r, np.float32).reshape(-1, d.H)
    T = r.shape[0]
    x = rmsnorm_bf16(r)
    ids0, _, _, _ = route(d, router, x)
    if callable(blobs):
        blobs = {int(e): blobs(int(e)) for e in np.unique(ids0)}
    arr, keep = _blob_table(d, blobs)
    sh = _c(shared, np.uint8) if d.has_shared else None
    r_out = np.empty((T, d.H), dtype=np.float64)
    xo = np.empty((T, d.H), dtype=np.uint16)
    y = np.empty((T, d.H), dtype=np.float64)
    ids = np.empty((T, d.K), dtype=np.int32)
    w = np.empty((T, d.K), dtype=np.float64)
    logits = np.empty((T, d.E), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    lib().or_residual_layer(ctypes.byref(d.c()), _p(router, _u16p), arr,
                            _p(sh, _u8p) if sh is not None else None, _p(r, _f32p), T,
                            _p(r_out, _f64p), _p(xo, _u16p), _p(y, _f64p), _p(ids, _i32p),
                            _p(w, _f64p), _p(logits, _f64p), _p(gap, _f64p))
    del keep
    return r_out, xo, y, ids, w, logits, gap
