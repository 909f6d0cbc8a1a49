"""Helpers for the GPU tests: a device-resident synthetic layer, host copies
of its exact bytes for the oracle, and the parity comparisons."""
from __future__ import annotations

import os

import numpy as np

import bit_dequant_expert_moe_amd as moe
import oracle
import synth

SHARED_ID = 0xFFFF  # generator expert index used for the shared expert

# the oracle's output rows on the host cores (same results for any count)
oracle.set_threads(min(16, os.cpu_count() or 1))

# Near-tie margin for routing: the fp32 router sums 4096 exact bf16 products
# per logit; with |W| ~ 0.02 and |x| ~ 1 the worst-case rounding bound is
# ~3e-4, so logits closer than 1e-3 in float64 may legitimately swap.
TIE_DELTA = 1e-3
# Output tolerance: max |y_gpu - y_oracle| <= 2e-3 * max |y_oracle|.
Y_TOL = 2e-3
W_TOL = 1e-5


class DeviceLayer:
    """One synthetic layer resident on the GPU."""

    def __init__(self, H, I, E, K, bits=4, has_shared=1, seed=1000, blob_seed=None, layer=0,
                 stride=None, z_range=None):
        import torch
        self.torch = torch
        self.dims = moe.Dims(hidden=H, inter=I, n_experts=E, top_k=K, bits=bits,
                             has_shared=has_shared)
        self.od = oracle.Dims(H=H, I=I, E=E, K=K, bits=bits, has_shared=has_shared)
        self.nbytes = moe.moe_expert_bytes(self.dims)
        self.stride = stride or self.nbytes
        self.params = synth.BlobParams(seed=blob_seed if blob_seed is not None else seed,
                                       H=H, I=I, bits=bits)
        if z_range is not None:
            self.params = synth.replace(self.params, z_lo=z_range[0], z_hi=z_range[1])
        self.layer = layer
        self.seed = seed
        self.experts = torch.empty(E * self.stride, dtype=torch.uint8, device="cuda")
        synth.gen_blobs_dev(self.params, layer, 0, E, self.experts.data_ptr(), self.stride,
                            torch.cuda.current_stream().cuda_stream)
        self.shared = None
        if has_shared:
            self.shared = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
            synth.gen_blobs_dev(self.params, layer, SHARED_ID, 1, self.shared.data_ptr(),
                                self.nbytes, torch.cuda.current_stream().cuda_stream)
        self.router_h = synth.router_weights(seed, layer, E, H)
        self.router = torch.from_numpy(self.router_h.view(np.int16)).cuda()
        self.L = moe.make_layer(self.router, self.experts, self.stride, self.shared)
        self._cache = {}

    def blob_host(self, e):
        """Host copy of the exact device bytes of expert e."""
        if e not in self._cache:
            t = self.experts[e * self.stride: e * self.stride + self.nbytes]
            self._cache[e] = t.cpu().numpy().copy()
        return self._cache[e]

    def shared_host(self):
        return self.shared.cpu().numpy().copy() if self.shared is not None else None

    def x_dev(self, x_u16):
        return self.torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).cuda()

    def decode(self, x_u16, T=None, want_logits=False):
        """moe_route (for logits) + moe_layer_decode; returns host arrays."""
        torch = self.torch
        x_u16 = np.ascontiguousarray(x_u16).reshape(-1, self.dims.hidden)
        T = x_u16.shape[0]
        xd = self.x_dev(x_u16)
        ws = moe.alloc_workspace(self.dims, T)
        y = torch.empty((T, self.dims.hidden), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, self.dims.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, self.dims.top_k), dtype=torch.float32, device="cuda")
        logits = None
        if want_logits:
            logits = torch.empty((T, self.dims.n_experts), dtype=torch.float32, device="cuda")
            ids2 = torch.empty_like(ids)
            w2 = torch.empty_like(w)
            moe.moe_route(self.dims, self.router, xd, T, ids2, w2, logits, ws)
        moe.moe_layer_decode(self.dims, self.L, xd, T, y, ids, w, ws)
        torch.cuda.synchronize()
        err = moe.moe_get_device_error(ws)
        out = dict(y=y.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy(), err=err)
        if want_logits:
            out["logits"] = logits.cpu().numpy()
        return out

    def decode_residual(self, r_f32, ws=None, outputs=True):
        """moe_layer_decode_residual on a copy of r; returns host arrays
        (x, y, ids, w only when outputs=True)."""
        torch = self.torch
        r_f32 = np.ascontiguousarray(r_f32, dtype=np.float32).reshape(-1, self.dims.hidden)
        T = r_f32.shape[0]
        rd = torch.from_numpy(r_f32.copy()).cuda()
        ws = ws if ws is not None else moe.alloc_workspace(self.dims, T)
        out = {}
        if outputs:
            x = torch.empty((T, self.dims.hidden), dtype=torch.int16, device="cuda")
            y = torch.empty((T, self.dims.hidden), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, self.dims.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, self.dims.top_k), dtype=torch.float32, device="cuda")
            moe.moe_layer_decode_residual(self.dims, self.L, rd, T, x, y, ids, w, ws)
        else:
            moe.moe_layer_decode_residual(self.dims, self.L, rd, T, ws=ws)
        torch.cuda.synchronize()
        out["err"] = moe.moe_get_device_error(ws)
        out["r"] = rd.cpu().numpy()
        if outputs:
            out.update(x=x.cpu().numpy().view(np.uint16), y=y.cpu().numpy(),
                       ids=ids.cpu().numpy(), w=w.cpu().numpy())
        return out
# The device sums r^2 in fp32 and scales in fp32, the oracle in float64: a
# value within ~1e-7 relative of a bf16 rounding boundary may round the other
# way (expected well under one element per 4096-vector).  Allowed: at most
# this many elements per vector, each one bf16 step away.
X_MISMATCH_MAX = 8


def check_norm(x_gpu, r):
    """x_gpu (bf16 bits [H]) against the oracle's RMS norm of r."""
    x_o = oracle.rmsnorm_bf16(np.asarray(r, np.float32))
    d = x_gpu.astype(np.int32) - x_o.astype(np.int32)
    bad = np.nonzero(d)[0]
    assert bad.size <= X_MISMATCH_MAX, "x differs from the oracle in %d elements" % bad.size
    assert np.all(np.abs(d) <= 1) and np.all((x_gpu[bad] ^ x_o[bad]) & 0x8000 == 0)
    return int(bad.size)


def check_routing(od, ids_gpu, w_gpu, logits_or, gap_or, K):
    """ids exact where the float64 gap >= TIE_DELTA; otherwise each chosen
    expert's float64 logit is within TIE_DELTA of the correct one at its rank.
    Weights are compared with the float64 softmax over the GPU's choice."""
    T = ids_gpu.shape[0]
    exact = 0
    for t in range(T):
        l = logits_or[t]
        srt = np.sort(l)[::-1][:K]
        order = np.lexsort((np.arange(l.size), -l))[:K]
        if gap_or[t] >= TIE_DELTA:
            np.testing.assert_array_equal(ids_gpu[t], order, err_msg="token %d" % t)
            exact += 1
        else:
            assert len(set(ids_gpu[t].tolist())) == K
            assert np.all(np.abs(l[ids_gpu[t]] - srt) <= TIE_DELTA), "token %d" % t
        sel = l[ids_gpu[t]]
        ww = np.exp(sel - sel.max())
        ww /= ww.sum()
        np.testing.assert_allclose(w_gpu[t], ww, rtol=0, atol=W_TOL)
        assert abs(float(np.sum(w_gpu[t], dtype=np.float64)) - 1.0) <= 1e-6
    return exact


def max_rel_err(y_gpu, y_or):
    """max_i |y_gpu - y_or| / max_i |y_or| per token (last axis), worst token."""
    y_gpu = np.atleast_2d(np.asarray(y_gpu, np.float64))
    y_or = np.atleast_2d(np.asarray(y_or, np.float64))
    num = np.max(np.abs(y_gpu - y_or), axis=-1)
    den = np.max(np.abs(y_or), axis=-1)
    return float(np.max(num / den))
