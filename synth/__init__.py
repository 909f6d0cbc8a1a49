"""Seeded synthetic inputs for the MoE layer (shared by the tests, the oracle
checks and the benchmark).

Holds no arithmetic of the method itself: it draws random expert blobs in the
library's storage format, random bf16 router matrices and random
RMS-normalised bf16 activations.

* Expert blobs come from a counter-based SplitMix64 hash of
  (seed, layer, expert, word index) implemented twice with identical results:
  ``gen_host.c`` (host) and ``gen_dev.hip`` (device, used to fill the
  hundreds of GB of a resident expert stack in place).
* Router matrices and activations come from numpy's PCG64 stream keyed by
  (seed, tag, layer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "gen_host.c")
_DEV_SRC = os.path.join(_HERE, "gen_dev.hip")
_COMMON = os.path.join(_HERE, "synth_common.h")
_HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
_DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _stale(lib, srcs):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(s) > t for s in srcs)


def build(force: bool = True, device: bool = True) -> None:
    """Compiles the host generator (gcc) and, if `device`, the HIP one."""
    if force or _stale(_HOST_LIB, [_HOST_SRC, _COMMON]):
        tmp = _HOST_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _HOST_SRC])
        os.replace(tmp, _HOST_LIB)
    if device and (force or _stale(_DEV_LIB, [_DEV_SRC, _COMMON])):
        tmp = _DEV_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([HIPCC, *HIP_FLAGS, "-ffp-contract=off", "-o", tmp, _DEV_SRC])
        os.replace(tmp, _DEV_LIB)


class _Params(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("s_lo", ctypes.c_float), ("s_hi", ctypes.c_float),
                ("z_lo", ctypes.c_float), ("z_hi", ctypes.c_float)]


@dataclass(frozen=True)
class BlobParams:
    """Distribution of synthetic expert blobs: codes uniform over all
    2^bits values, scale ~ U(s_lo, s_hi), bias ~ U(z_lo, z_hi), both bf16."""
    seed: int
    H: int = 4096
    I: int = 1024
    bits: int = 4
    s_lo: float = 0.005
    s_hi: float = 0.02
    z_lo: float = -0.08
    z_hi: float = 0.08

    def c(self) -> _Params:
        return _Params(self.seed, self.H, self.I, self.bits, self.s_lo, self.s_hi,
                       self.z_lo, self.z_hi)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        build(force=False, device=False)
        L = ctypes.CDLL(_HOST_LIB)
        L.synth_blob_words.restype = ctypes.c_uint64
        L.synth_blob_words.argtypes = [ctypes.c_int32] * 3
        L.synth_gen_blob_host.restype = None
        L.synth_gen_blob_host.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_void_p]
        L.synth_gen_words_host.restype = None
        L.synth_gen_words_host.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint32,
                                           ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                           ctypes.c_void_p]
        _host = L
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_LIB):
            raise RuntimeError("synth/libsynth_dev.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_DEV_LIB)
        L.synth_gen_blobs_dev.restype = ctypes.c_int
        L.synth_gen_blobs_dev.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
        _dev = L
    return _dev


def blob_bytes(p: BlobParams) -> int:
    return 4 * int(_host_lib().synth_blob_words(p.H, p.I, p.bits))


def blob_host(p: BlobParams, layer: int, expert: int) -> np.ndarray:
    """The blob of (layer, expert) as host uint8."""
    n = blob_bytes(p) // 4
    out = np.empty(n, dtype=np.uint32)
    cp = p.c()
    _host_lib().synth_gen_blob_host(ctypes.byref(cp), layer, expert, out.ctypes.data)
    return out.view(np.uint8)


def words_host(p: BlobParams, layer: int, expert: int, w0: int, n: int) -> np.ndarray:
    """Words [w0, w0+n) of the blob of (layer, expert) as uint32."""
    out = np.empty(n, dtype=np.uint32)
    cp = p.c()
    _host_lib().synth_gen_words_host(ctypes.byref(cp), layer, expert, w0, n, out.ctypes.data)
    return out


def gen_blobs_dev(p: BlobParams, layer: int, e0: int, n: int, dst_ptr: int, stride: int,
                  stream_ptr: int = 0) -> None:
    """Fills n blobs (experts e0..e0+n-1 of `layer`) at device address dst_ptr
    with `stride` bytes between blobs, enqueued on stream_ptr."""
    cp = p.c()
    rc = _dev_lib().synth_gen_blobs_dev(ctypes.byref(cp), layer, e0, n, ctypes.c_void_p(dst_ptr),
                                        stride, ctypes.c_void_p(stream_ptr))
    if rc != 0:
        raise RuntimeError("synth_gen_blobs_dev failed with %d" % rc)


# ---- bf16 and activations ------------------------------------------------------

def f32_to_bf16(a) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_TAG_ROUTER, _TAG_X, _TAG_NOISE, _TAG_RESID = 1, 2, 3, 4


def router_weights(seed: int, layer: int, E: int, H: int, std: float = 0.02) -> np.ndarray:
    """bf16 [E][H] with entries ~ N(0, std^2)."""
    g = np.random.default_rng([seed, _TAG_ROUTER, layer])
    return f32_to_bf16(g.standard_normal((E, H)) * std)


def rms_normalise(z: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Plain RMS normalisation along the last axis (no gain)."""
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def tokens(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    """T independent activations ~ N(0,1), RMS-normalised, bf16 [T][H]."""
    g = np.random.default_rng([seed, _TAG_X, layer])
    return f32_to_bf16(rms_normalise(g.standard_normal((T, H))))


def tokens_ar1(seed: int, layer: int, T: int, H: int, rho: float) -> np.ndarray:
    """T consecutive activations of one layer with an AR(1) correlation rho
    from token to token (z_t = rho z_{t-1} + sqrt(1 - rho^2) e_t, e_t ~ N(0,1)),
    RMS-normalised, bf16 [T][H].  rho sets how often consecutive tokens pick
    the same experts."""
    g = np.random.default_rng([seed, _TAG_NOISE, layer])
    z = np.empty((T, H), dtype=np.float64)
    z[0] = g.standard_normal(H)
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, T):
        z[t] = rho * z[t - 1] + c * g.standard_normal(H)
    return f32_to_bf16(rms_normalise(z))


def residual(seed: int, T: int, H: int, rho: float = 0.0, outliers: int = 4,
             outlier_scale: float = 20.0) -> np.ndarray:
    """T consecutive residual-stream vectors, fp32 [T][H]: N(0,1) per channel,
    AR(1)-correlated with coefficient rho from token to token, with
    `outliers` fixed channels scaled by `outlier_scale` (residual streams of
    large transformers carry a few channels far above the rest; the value is
    a stand-in, not a measurement).  Not normalised."""
    g = np.random.default_rng([seed, _TAG_RESID, 0])
    big = g.choice(H, size=outliers, replace=False) if outliers else np.zeros(0, np.int64)
    z = np.empty((T, H), dtype=np.float64)
    z[0] = g.standard_normal(H)
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, T):
        z[t] = rho * z[t - 1] + c * g.standard_normal(H)
    z[:, big] *= outlier_scale
    return z.astype(np.float32)


from .workloads import WORKLOADS, Workload  # noqa: E402,F401
