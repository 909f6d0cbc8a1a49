"""GPU parity of moe_layer_decode_residual -- RMS norm of the residual, the
MoE layer, residual add -- against the float64 oracle, through the C ABI.

Bar per token: x within one bf16 step of the oracle's norm at no more than a
handful of elements (fp32 against float64 sums of squares, see gpu_util);
routing and y as for moe_layer_decode, teacher-forced on the x the kernel
formed; the updated residual equal to r + y in fp32, bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_dequant_expert_moe_amd as moe  # noqa: E402


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def layers():
    # two full 512-expert layers (layers 0 and 1 of one stack) with zero-mean
    # weight matrices, so that a chain of them stays non-degenerate
    return [gu.DeviceLayer(4096, 1024, 512, 4, bits=4, seed=1005, layer=l,
                           z_range=synth.workloads.CENTRED_Z) for l in range(2)]


def _check_step(L, r_before, out, t, label):
    """One token t of one call: norm, routing, y, residual."""
    nx = gu.check_norm(out["x"][t], r_before[t])
    x = out["x"][t:t + 1]
    _, _, logits_o, gap_o = oracle.route(L.od, L.router_h, x)
    gu.check_routing(L.od, out["ids"][t:t + 1], out["w"][t:t + 1], logits_o, gap_o, L.dims.top_k)
    sel = logits_o[0][out["ids"][t]]
    wf = np.exp(sel - sel.max())
    wf /= wf.sum()
    y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x, out["ids"][t:t + 1],
                                wf[None])
    err = gu.max_rel_err(out["y"][t][None], y_o)
    _say("  %s token %d: x mismatches %d, max|dy|/max|y| = %.3e" % (label, t, nx, err))
    assert err <= gu.Y_TOL
    np.testing.assert_array_equal(out["r"][t], (r_before[t] + out["y"][t]).astype(np.float32))


def test_residual_chain_fused(layers):
    # three chained calls (layers 0, 1, 0) on one workspace, one token
    r = synth.residual(1005, 1, 4096)
    ws = moe.alloc_workspace(layers[0].dims, 1)
    for step, l in enumerate([0, 1, 0]):
        _say("residual chain step", step, "layer", l)
        out = layers[l].decode_residual(r, ws=ws)
        assert out["err"] == 0
        _check_step(layers[l], r, out, 0, "chain step %d" % step)
        # the layer moves the residual (the chain is not degenerate)
        assert np.sqrt(np.mean(out["y"][0].astype(np.float64) ** 2)) > 1.0
        r = out["r"]


def test_residual_matches_oracle_residual_layer(layers):
    # not teacher-forced: the oracle forms x itself (float64 norm), routes and
    # combines; away from float64 near-ties the ids agree and r_out is within
    # the output tolerance of y
    L = layers[0]
    r = synth.residual(1006, 1, 4096)
    out = L.decode_residual(r)
    r_o, x_o, y_o, ids_o, w_o, logits_o, gap_o = oracle.residual_layer(
        L.od, L.router_h, L.blob_host, L.shared_host(), r)
    if gap_o[0] >= gu.TIE_DELTA:
        np.testing.assert_array_equal(out["ids"][0], ids_o[0])
        assert np.max(np.abs(out["r"][0] - r_o[0])) <= gu.Y_TOL * np.max(np.abs(y_o[0]))


def test_residual_outputs_optional_and_deterministic(layers):
    L = layers[1]
    r = synth.residual(1007, 1, 4096)
    a = L.decode_residual(r)
    b = L.decode_residual(r, outputs=False)
    c = L.decode_residual(r)
    assert a["err"] == b["err"] == c["err"] == 0
    np.testing.assert_array_equal(a["r"], b["r"])
    np.testing.assert_array_equal(a["r"], c["r"])
    np.testing.assert_array_equal(a["x"], c["x"])


def test_residual_multi_token(layers):
    # T=5 takes the norm kernel, the router, the grouped expert GEMMs and the
    # residual add kernel
    L = layers[0]
    r = synth.residual(1008, 5, 4096, rho=0.5)
    out = L.decode_residual(r)
    assert out["err"] == 0
    for t in range(5):
        _check_step(L, r, out, t, "T=5")


def test_residual_2bit_and_no_shared():
    for bits, has_shared, seed in [(2, 1, 1009), (4, 0, 1010)]:
        L = gu.DeviceLayer(4096, 1024, 64, 4, bits=bits, has_shared=has_shared, seed=seed)
        r = synth.residual(seed, 1, 4096)
        out = L.decode_residual(r)
        assert out["err"] == 0
        _check_step(L, r, out, 0, "bits %d shared %d" % (bits, has_shared))


def test_residual_small_scale_and_outliers(layers):
    # the norm removes the scale: r and 1e-3 r give the same routing away from
    # ties, and an r with huge outlier channels still meets the bar
    L = layers[1]
    r = synth.residual(1011, 1, 4096, outliers=8, outlier_scale=300.0)
    out = L.decode_residual(r)
    _check_step(L, r, out, 0, "outliers x300")
    out2 = L.decode_residual(r * np.float32(1e-3))
    _check_step(L, r * np.float32(1e-3), out2, 0, "scaled 1e-3")


def test_residual_graph_replay_matches_eager(layers):
    # a captured chain of the two layers with the residual restored inside the
    # graph (a device copy, no memset), replayed with eager work in between
    r0 = torch.from_numpy(synth.residual(1012, 1, 4096)).cuda()
    r = torch.empty_like(r0)
    ws = moe.alloc_workspace(layers[0].dims, 1)
    r.copy_(r0)
    for L in layers:
        moe.moe_layer_decode_residual(L.dims, L.L, r, 1, ws=ws)
    torch.cuda.synchronize()
    want = r.cpu().numpy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            r.copy_(r0)
            for L in layers:
                moe.moe_layer_decode_residual(L.dims, L.L, r, 1, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        r.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r.cpu().numpy(), want)
        moe.moe_layer_decode_residual(layers[0].dims, layers[0].L, r, 1, ws=ws)
        torch.cuda.synchronize()
    assert moe.moe_get_device_error(ws) == 0
