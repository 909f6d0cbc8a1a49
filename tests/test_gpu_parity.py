"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Bar: routed ids exact (away from float64 near-ties, see gpu_util), routing
weights within 1e-5, dequantised weights bit-exact, outputs within
2e-3 * max|oracle| (fp32 accumulation on the device)."""
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
def tiny():
    # one layer, 16 experts, hidden 4096, intermediate 1024, top-4 + shared
    return gu.DeviceLayer(4096, 1024, 16, 4, bits=4, seed=1000)


@pytest.fixture(scope="module")
def full():
    # one full layer, 512 experts
    return gu.DeviceLayer(4096, 1024, 512, 4, bits=4, seed=1001)


# ---- generator and dequantisation -----------------------------------------------

@pytest.mark.parametrize("bits", [4, 2])
def test_device_generator_matches_host(bits):
    L = gu.DeviceLayer(4096, 1024, 4, 2, bits=bits, seed=42)
    for e in [0, 3]:
        np.testing.assert_array_equal(L.blob_host(e), synth.blob_host(L.params, 0, e))
    np.testing.assert_array_equal(L.shared_host(), synth.blob_host(L.params, 0, gu.SHARED_ID))


DECODERS = [("scalar", moe.DEQ_SCALAR), ("fp16 pair", moe.DEQ_FP16_PAIR),
            ("fp8 pair", moe.DEQ_FP8_PAIR), ("bf16 pair", moe.DEQ_BF16_PAIR),
            ("bf16 slice", moe.DEQ_BF16_SLICE)]


def _dequant_dev(L, blob_dev, which, decoder=None):
    rows, cols = (L.dims.hidden, L.dims.inter) if which == 2 else (L.dims.inter, L.dims.hidden)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    if decoder is None:
        moe.moe_dequantize(L.dims, blob_dev, which, out)
    else:
        moe.moe_dequantize_as(L.dims, blob_dev, which, decoder, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("shape", [(4096, 1024, 4), (4096, 1024, 2), (256, 512, 4), (1024, 256, 2)])
def test_dequantize_bit_exact(shape):
    # every decoder the kernels use (the unpack function each kernel calls),
    # on every matrix, against the oracle's one rounding of s q + z
    H, I, bits = shape
    _say("dequant", shape)
    L = gu.DeviceLayer(H, I, 3, 2, bits=bits, seed=7)
    for e in [0, 2]:
        blob_dev = L.experts[e * L.stride:]
        for which in range(3):
            want = oracle.dequant_matrix_f32(L.od, L.blob_host(e), which).view(np.uint32)
            got = _dequant_dev(L, blob_dev, which)
            np.testing.assert_array_equal(got.view(np.uint32), want)
            for name, dec in DECODERS:
                got = _dequant_dev(L, blob_dev, which, dec)
                np.testing.assert_array_equal(got.view(np.uint32), want,
                                              err_msg="%s, matrix %d" % (name, which))


def test_dequantize_shared_tiny(tiny):
    for which in range(3):
        want = oracle.dequant_matrix_f32(tiny.od, tiny.shared_host(), which).view(np.uint32)
        for name, dec in DECODERS:
            got = _dequant_dev(tiny, tiny.shared, which, dec)
            np.testing.assert_array_equal(got.view(np.uint32), want, err_msg=name)


# ---- routing ------------------------------------------------------------------

# T >= 512 takes the 64 x 64 tiled router (600 tokens and the tiny layer's 16
# experts: ragged in both; 1024 tokens: split along the hidden dimension)
@pytest.mark.parametrize("which,T", [("tiny", 1), ("tiny", 37), ("full", 1), ("full", 64),
                                     ("tiny", 600), ("full", 1024)])
def test_route_parity(which, T, tiny, full):
    L = tiny if which == "tiny" else full
    _say("route", which, T)
    x = synth.tokens(L.seed + 17, 0, T, 4096)
    out = L.decode(x, want_logits=True)
    ids_o, w_o, logits_o, gap_o = oracle.route(L.od, L.router_h, x)
    # logits: fp32 sums of exact products vs float64
    assert np.max(np.abs(out["logits"] - logits_o)) < 1e-4
    exact = gu.check_routing(L.od, out["ids"], out["w"], logits_o, gap_o, L.dims.top_k)
    _say("  tokens with exact ids:", exact, "of", T)
    assert exact >= 0.8 * T


@pytest.mark.parametrize("E,K,T", [(1000, 8, 520), (100, 4, 513), (64, 2, 4096)])
def test_route_parity_tiled_ragged(E, K, T):
    # the 64 x 64 tiled router (T >= 512) with expert counts off its tiles
    # (1000 and 100: a partial last tile; 64: one tile) and K up to 8: logits
    # within 1e-4 of float64, ids and weights as in the other routing tests;
    # only the router is needed
    import torch
    H = 4096
    dims = moe.Dims(hidden=H, inter=1024, n_experts=E, top_k=K)
    od = oracle.Dims(H=H, I=1024, E=E, K=K)
    router_h = synth.router_weights(2000 + E, 0, E, H)
    x_h = synth.tokens(2000 + E, 1, T, H)
    _say("route tiled", E, K, T)
    r = torch.from_numpy(router_h.view(np.int16)).cuda()
    x = torch.from_numpy(x_h.view(np.int16)).cuda()
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(dims, T)
    moe.moe_route(dims, r, x, T, ids, w, logits, ws)
    torch.cuda.synchronize()
    ids_o, w_o, logits_o, gap_o = oracle.route(od, router_h, x_h)
    assert np.max(np.abs(logits.cpu().numpy() - logits_o)) < 1e-4
    exact = gu.check_routing(od, ids.cpu().numpy(), w.cpu().numpy(), logits_o, gap_o, K)
    _say("  tokens with exact ids:", exact, "of", T)
    assert exact >= 0.8 * T


# ---- full layer -----------------------------------------------------------------

def _layer_check(L, x, label):
    out = L.decode(x, want_logits=True)
    T = x.shape[0]
    ids_o, w_o, logits_o, gap_o = oracle.route(L.od, L.router_h, x)
    gu.check_routing(L.od, out["ids"], out["w"], logits_o, gap_o, L.dims.top_k)
    # teacher-forced: the oracle combines the experts the GPU picked, with the
    # float64 weights of that pick
    w_for_gpu = np.empty_like(out["w"], dtype=np.float64)
    for t in range(T):
        sel = logits_o[t][out["ids"][t]]
        ww = np.exp(sel - sel.max())
        w_for_gpu[t] = ww / ww.sum()
    y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x, out["ids"], w_for_gpu)
    err = gu.max_rel_err(out["y"], y_o)
    _say("  %s: max|dy|/max|y| = %.3e" % (label, err))
    assert err <= gu.Y_TOL
    assert out["err"] == 0
    return out


def test_layer_decode_tiny(tiny):
    x = synth.tokens(1000, 0, 1, 4096)
    _layer_check(tiny, x, "tiny T=1")


def test_layer_decode_full(full):
    x = synth.tokens(1001, 0, 1, 4096)
    _layer_check(full, x, "full T=1")


def test_layer_decode_full_batch(full):
    x = synth.tokens(1001, 5, 4, 4096)
    _layer_check(full, x, "full T=4")


def test_layer_decode_full_T64(full):
    # the batched workload: 64 tokens, 512 experts; pairs grouped by expert
    x = synth.tokens(1003, 0, 64, 4096)
    _layer_check(full, x, "full T=64")


@pytest.mark.parametrize("bits", [4, 2])
def test_grouped_buckets_over_one_chunk(bits):
    # E = K = 4: every token selects every expert, so each bucket holds all 64
    # tokens (two 32-pair chunks), and the shared bucket too
    L = gu.DeviceLayer(1024, 512, 4, 4, bits=bits, seed=77 + bits)
    x = synth.tokens(77, 0, 64, 1024)
    _layer_check(L, x, "E=K=4 T=64 %d-bit" % bits)


def test_grouped_2bit_full_T16():
    L = gu.DeviceLayer(4096, 1024, 512, 4, bits=2, seed=1001, blob_seed=1004)
    x = synth.tokens(1001, 3, 16, 4096)
    _layer_check(L, x, "2-bit full T=16")


def test_layer_decode_2bit_tiny():
    L = gu.DeviceLayer(4096, 1024, 16, 4, bits=2, seed=1000, blob_seed=1004)
    x = synth.tokens(1000, 0, 2, 4096)
    _layer_check(L, x, "2-bit tiny T=2")


@pytest.mark.parametrize("cfg", [
    (256, 256, 8, 2, 4, 1), (512, 2048, 32, 8, 4, 1), (1024, 256, 4, 4, 2, 0),
    (8192, 512, 64, 1, 4, 1), (2048, 4096, 16, 3, 2, 1), (16384, 256, 2, 2, 4, 1),
    # expert counts off the 16-row router tiles; 1000 experts take the fused
    # kernel's four router rows per workgroup, with rows past E
    (4096, 1024, 100, 4, 4, 1), (4096, 1024, 1000, 4, 4, 1), (4096, 1024, 1000, 4, 2, 0)])
def test_layer_decode_shapes(cfg):
    # one and three tokens (the single-token kernels, once per token, where
    # they cover the shape; else the three-kernel and the grouped path) and
    # four (the grouped path)
    H, I, E, K, bits, sh = cfg
    _say("shape", cfg)
    L = gu.DeviceLayer(H, I, E, K, bits=bits, has_shared=sh, seed=300 + H + I + E)
    for T in (1, 3, 4):
        x = synth.tokens(L.seed, T, T, H)
        _layer_check(L, x, "shape %s T=%d" % (cfg, T))


def test_expert_stride_padding():
    # experts placed at a stride larger than the blob
    L = gu.DeviceLayer(1024, 512, 8, 2, bits=4, seed=55, stride=2 * 1024 * 1024)
    x = synth.tokens(55, 0, 2, 1024)
    _layer_check(L, x, "padded stride")


# ---- expert forward with given routing ----------------------------------------------

def test_expert_forward_given_ids_and_invalid_id(tiny):
    L = tiny
    x = synth.tokens(999, 0, 2, 4096)
    ids = np.array([[3, 9, 1, 12], [15, 0, 7, 9999]], np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], np.float32)
    ws = moe.alloc_workspace(L.dims, 2)
    y = torch.empty((2, 4096), dtype=torch.float32, device="cuda")
    moe.moe_expert_forward(L.dims, L.L, L.x_dev(x), 2, torch.from_numpy(ids).cuda(),
                           torch.from_numpy(w).cuda(), y, ws)
    torch.cuda.synchronize()
    err = moe.moe_get_device_error(ws)
    assert err == 1  # the out-of-range id was reported
    assert moe.moe_get_device_error(ws) == 0  # and cleared
    y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x, ids,
                                w.astype(np.float64))
    assert gu.max_rel_err(y.cpu().numpy(), y_o) <= gu.Y_TOL


def test_expert_forward_repeated_ids_large_bucket(full):
    # the grouped path with a token that names one expert in three slots:
    # 2048 tokens x 3 slots put 6144 pairs (384 chunks of 16) in one bucket,
    # beyond what an 8-bit chunk field of a work item could index
    L = full
    T = 2048
    x = synth.tokens(1021, 0, T, 4096)
    rng = np.random.default_rng(5)
    ids = np.empty((T, 4), np.int32)
    ids[:, :3] = 5
    ids[:, 3] = rng.integers(0, 512, T)
    w = rng.dirichlet(np.ones(4), T).astype(np.float32)
    ws = moe.alloc_workspace(L.dims, T)
    y = torch.empty((T, 4096), dtype=torch.float32, device="cuda")
    moe.moe_expert_forward(L.dims, L.L, L.x_dev(x), T, torch.from_numpy(ids).cuda(),
                           torch.from_numpy(w).cuda(), y, ws)
    torch.cuda.synchronize()
    assert moe.moe_get_device_error(ws) == 0
    yh = y.cpu().numpy()
    for t in (0, 1, 777, 2047):
        y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x[t:t + 1],
                                    ids[t:t + 1], w[t:t + 1].astype(np.float64))
        err = gu.max_rel_err(yh[t], y_o)
        _say("  repeated ids, token %d: max|dy|/max|y| = %.2e" % (t, err))
        assert err <= gu.Y_TOL


# ---- invariants ---------------------------------------------------------------------

def test_batched_equals_single_and_deterministic(full):
    # same inputs -> bitwise-identical outputs, for the multi-token and the
    # single-token kernels; the two paths agree on ids (away from float64
    # near-ties) and on y within the output tolerance
    x = synth.tokens(1001, 9, 8, 4096)
    ob = full.decode(x)
    ob2 = full.decode(x)
    np.testing.assert_array_equal(ob["y"], ob2["y"])
    _, _, logits_o, gap_o = oracle.route(full.od, full.router_h, x)
    for t in range(8):
        o1 = full.decode(x[t:t + 1])
        o1b = full.decode(x[t:t + 1])
        np.testing.assert_array_equal(o1["y"], o1b["y"])
        if gap_o[t] >= gu.TIE_DELTA:
            np.testing.assert_array_equal(o1["ids"][0], ob["ids"][t])
            assert gu.max_rel_err(o1["y"][0], ob["y"][t]) <= gu.Y_TOL


def test_zero_filled_workspace_needs_no_init(full):
    # a zero-filled workspace is an initialised one: the same outputs bit for
    # bit as a workspace set up by moe_workspace_init (one token: the fused
    # kernel; eight tokens: the grouped path)
    import torch
    for T in (1, 8):
        x = full.x_dev(synth.tokens(1001, 70 + T, T, 4096))
        outs = []
        for zero in (False, True):
            if zero:
                n = moe.moe_workspace_bytes(full.dims, T)
                buf = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
                off = (-buf.data_ptr()) % 256
                ws = buf[off:off + n]
            else:
                ws = moe.alloc_workspace(full.dims, T)
            y = torch.empty((T, 4096), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, 4), dtype=torch.int32, device="cuda")
            for _ in range(2):  # first call and a second on the same workspace
                moe.moe_layer_decode(full.dims, full.L, x, T, y, ids, None, ws)
                torch.cuda.synchronize()
                assert moe.moe_get_device_error(ws) == 0
                outs.append((y.cpu().numpy().copy(), ids.cpu().numpy().copy()))
        for a, b in zip(outs[:2], outs[2:]):
            np.testing.assert_array_equal(a[0], b[0])
            np.testing.assert_array_equal(a[1], b[1])


# ---- single-token fused path: repeated calls, graphs, error word ----------------

@pytest.mark.parametrize("T", [2, 3])
def test_small_batches_run_per_token(full, T):
    # calls of up to three tokens run the single-token kernel once per token:
    # bitwise equal to T one-token calls, and within tolerance of the oracle
    x = synth.tokens(1004, T, T, 4096)
    ob = _layer_check(full, x, "full T=%d" % T)
    for t in range(T):
        o1 = full.decode(x[t:t + 1])
        np.testing.assert_array_equal(o1["ids"][0], ob["ids"][t])
        np.testing.assert_array_equal(o1["w"][0], ob["w"][t])
        np.testing.assert_array_equal(o1["y"][0], ob["y"][t])


def test_fused_consecutive_tokens_same_workspace(full):
    # 12 tokens decoded one call at a time on one workspace (the single-token
    # kernel's epoch advances per call) against the oracle, and against the
    # multi-token path on the same tokens for the routing
    L = full
    x = synth.tokens_ar1(1001, 3, 12, 4096, 0.97)
    ws = moe.alloc_workspace(L.dims, 1)
    xd = L.x_dev(x)
    ys, idss = [], []
    for t in range(12):
        y = torch.empty(4096, dtype=torch.float32, device="cuda")
        ids = torch.empty(4, dtype=torch.int32, device="cuda")
        w = torch.empty(4, dtype=torch.float32, device="cuda")
        moe.moe_layer_decode(L.dims, L.L, xd[t], 1, y, ids, w, ws)
        ys.append(y)
        idss.append((ids, w))
    torch.cuda.synchronize()
    assert moe.moe_get_device_error(ws) == 0
    ids_o, w_o, logits_o, gap_o = oracle.route(L.od, L.router_h, x)
    ids_g = np.stack([i.cpu().numpy() for i, _ in idss])
    w_g = np.stack([w.cpu().numpy() for _, w in idss])
    gu.check_routing(L.od, ids_g, w_g, logits_o, gap_o, 4)
    for t in [0, 5, 11]:
        sel = logits_o[t][ids_g[t]]
        wf = np.exp(sel - sel.max())
        wf /= wf.sum()
        y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x[t:t + 1], ids_g[t:t + 1],
                                    wf[None])
        err = gu.max_rel_err(ys[t].cpu().numpy()[None], y_o)
        _say("  fused token %d: max|dy|/max|y| = %.3e" % (t, err))
        assert err <= gu.Y_TOL


def test_fused_graph_replay_matches_eager(full):
    L = full
    x = synth.tokens(1001, 21, 3, 4096)
    xd = L.x_dev(x)
    ws = moe.alloc_workspace(L.dims, 1)
    y_e = torch.empty((3, 4096), dtype=torch.float32, device="cuda")
    for t in range(3):
        moe.moe_layer_decode(L.dims, L.L, xd[t], 1, y_e[t], ws=ws)
    torch.cuda.synchronize()
    y_g = torch.zeros((3, 4096), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(3):
                moe.moe_layer_decode(L.dims, L.L, xd[t], 1, y_g[t], ws=ws)
    torch.cuda.synchronize()
    for rep in range(5):
        y_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y_g.cpu().numpy(), y_e.cpu().numpy())
        # eager work between replays on the same workspace
        moe.moe_layer_decode(L.dims, L.L, xd[0], 1, y_e[0], ws=ws)
        torch.cuda.synchronize()
    assert moe.moe_get_device_error(ws) == 0


def test_fused_given_ids_single_token(tiny):
    L = tiny
    x = synth.tokens(4242, 0, 1, 4096)
    for ids_row, err_want in [([3, 9, 1, 12], 0), ([15, 0, 7, -1], 1)]:
        ids = np.array([ids_row], np.int32)
        w = np.array([[0.4, 0.3, 0.2, 0.1]], np.float32)
        ws = moe.alloc_workspace(L.dims, 1)
        y = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
        moe.moe_expert_forward(L.dims, L.L, L.x_dev(x), 1, torch.from_numpy(ids).cuda(),
                               torch.from_numpy(w).cuda(), y, ws)
        torch.cuda.synchronize()
        assert moe.moe_get_device_error(ws) == err_want
        y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x, ids,
                                    w.astype(np.float64))
        assert gu.max_rel_err(y.cpu().numpy(), y_o) <= gu.Y_TOL


def test_fused_2bit_single_token():
    L = gu.DeviceLayer(4096, 1024, 64, 4, bits=2, seed=1000, blob_seed=1004)
    for t in range(3):
        x = synth.tokens(1000, 40 + t, 1, 4096)
        _layer_check(L, x, "2-bit fused token %d" % t)


def test_fused_no_shared_expert():
    L = gu.DeviceLayer(4096, 1024, 64, 4, bits=4, has_shared=0, seed=777)
    for t in range(3):
        x = synth.tokens(777, 10 + t, 1, 4096)
        _layer_check(L, x, "fused, no shared expert, token %d" % t)


# ---- prefill chunks: many tokens per call ----------------------------------------

@pytest.mark.parametrize("T", [1024, 4096])
def test_prefill_chunk_sampled(full, T):
    # all 512 experts in play, the shared expert's bucket holds T pairs
    # (T / 16 work items); sampled tokens against the oracle, teacher-forced
    x = synth.tokens(1001, 40 + T, T, 4096)
    out = full.decode(x)
    assert out["err"] == 0
    sample = sorted({0, 1, T // 3, T // 2, T - 2, T - 1})
    _, _, logits_o, gap_o = oracle.route(full.od, full.router_h, x[sample])
    gu.check_routing(full.od, out["ids"][sample], out["w"][sample], logits_o, gap_o, 4)
    wf = np.empty((len(sample), 4))
    for i, t in enumerate(sample):
        sel = logits_o[i][out["ids"][t]]
        e = np.exp(sel - sel.max())
        wf[i] = e / e.sum()
    y_o = oracle.expert_forward(full.od, full.blob_host, full.shared_host(), x[sample],
                                out["ids"][sample], wf)
    err = gu.max_rel_err(out["y"][sample], y_o)
    _say("  prefill T=%d, %d sampled tokens: max|dy|/max|y| = %.3e" % (T, len(sample), err))
    assert err <= gu.Y_TOL
    # every token's row is finite and the routing uses many experts
    assert np.isfinite(out["y"]).all()
    assert len(np.unique(out["ids"])) > 400
