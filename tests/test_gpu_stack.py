"""GPU parity of consecutive layers of a resident stack, as the decode
benchmark runs them: 8 full 512-expert layers per token, one call per layer
on one workspace, captured in a graph per token and replayed.  Every layer of
every checked token is compared with the float64 oracle: routing exact away
from near-ties, y within 2e-3 max|y| (teacher-forced on the x and the routing
the GPU used).  On the chained stack x of each layer is the RMS norm of the
residual, which every layer updates (r += y): x is checked against the
oracle's norm of the residual the GPU held before the layer, and the final
residual against r + y summed in fp32 on the host."""
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

N_LAYERS = 8
N_TOK = 3


def _say(*a):
    print(*a, flush=True)


def _stack(chain):
    z = synth.workloads.CENTRED_Z if chain else None
    return [gu.DeviceLayer(4096, 1024, 512, 4, bits=4, seed=1002, layer=l, z_range=z)
            for l in range(N_LAYERS)]


@pytest.fixture(scope="module")
def plain_stack():
    return _stack(False)


@pytest.fixture(scope="module")
def chain_stack():
    return _stack(True)


def _oracle_layer_check(L, x, ids, w, y, label):
    _, _, logits_o, gap_o = oracle.route(L.od, L.router_h, x[None])
    gu.check_routing(L.od, ids[None], w[None], logits_o, gap_o, L.dims.top_k)
    sel = logits_o[0][ids]
    wf = np.exp(sel - sel.max())
    wf /= wf.sum()
    y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x[None], ids[None], wf[None])
    err = gu.max_rel_err(y, y_o)
    _say("  %s: ids %s, max|dy|/max|y| = %.2e" % (label, ids.tolist(), err))
    assert err <= gu.Y_TOL
    return err


class _Run:
    """Device buffers of N_TOK tokens through the stack; `fused` runs each
    token as one moe_stack_decode(_residual) call, else one single-layer call
    per layer."""

    def __init__(self, layers, chain, fused=False):
        self.layers, self.chain, self.fused = layers, chain, fused
        self.arr = moe.layer_array([L.L for L in layers])
        self.dims = layers[0].dims
        H = 4096
        if chain:
            self.r0_h = synth.residual(1002, N_TOK, H, 0.97)
            self.r0 = torch.from_numpy(self.r0_h).cuda()
            self.r = torch.empty_like(self.r0)
            self.x = torch.zeros((N_TOK, N_LAYERS, H), dtype=torch.int16, device="cuda")
        else:
            self.x_h = np.stack([synth.tokens_ar1(1002, l, N_TOK, H, 0.97)
                                 for l in range(N_LAYERS)], axis=1)
            self.x = torch.from_numpy(self.x_h.view(np.int16)).cuda()
        self.y = torch.zeros((N_TOK, N_LAYERS, H), dtype=torch.float32, device="cuda")
        self.ids = torch.zeros((N_TOK, N_LAYERS, 4), dtype=torch.int32, device="cuda")
        self.w = torch.zeros((N_TOK, N_LAYERS, 4), dtype=torch.float32, device="cuda")
        self.ws = moe.alloc_workspace(self.dims, 1)
        self.wsb = self.ws.numel()

    def enqueue(self, t, sp):
        if self.chain:
            self.r[t].copy_(self.r0[t])
        if self.fused:
            if self.chain:
                moe.moe_stack_decode_residual(self.dims, self.arr, self.r[t], self.x[t], self.y[t],
                                              self.ids[t], self.w[t], self.ws, self.wsb, sp)
            else:
                moe.moe_stack_decode(self.dims, self.arr, self.x[t], self.y[t], self.ids[t],
                                     self.w[t], self.ws, self.wsb, sp)
            return
        for l, L in enumerate(self.layers):
            if self.chain:
                moe.moe_layer_decode_residual(self.dims, L.L, self.r[t], 1, self.x[t, l],
                                              self.y[t, l], self.ids[t, l], self.w[t, l],
                                              self.ws, self.wsb, sp)
            else:
                moe.moe_layer_decode(self.dims, L.L, self.x[t, l], 1, self.y[t, l],
                                     self.ids[t, l], self.w[t, l], self.ws, self.wsb, sp)

    def host(self):
        out = dict(y=self.y.cpu().numpy(), ids=self.ids.cpu().numpy(), w=self.w.cpu().numpy(),
                   x=self.x.cpu().numpy().view(np.uint16))
        if self.chain:
            out["r"] = self.r.cpu().numpy()
        return out


def _check_stack(run, out):
    worst = 0.0
    for t in range(N_TOK):
        r = run.r0_h[t].copy() if run.chain else None
        for l, L in enumerate(run.layers):
            x = out["x"][t, l]
            if run.chain:
                gu.check_norm(x, r)
            worst = max(worst, _oracle_layer_check(L, x, out["ids"][t, l], out["w"][t, l],
                                                   out["y"][t, l], "token %d layer %d" % (t, l)))
            if run.chain:
                r = (r + out["y"][t, l]).astype(np.float32)
        if run.chain:
            # the residual after the last layer is r + y of every layer, in fp32
            np.testing.assert_array_equal(out["r"][t], r)
    return worst


def _eager(run):
    sp = torch.cuda.current_stream().cuda_stream
    for t in range(N_TOK):
        run.enqueue(t, sp)
    torch.cuda.synchronize()
    assert moe.moe_get_device_error(run.ws) == 0
    return run.host()


@pytest.mark.parametrize("chain", [False, True], ids=["plain", "chain"])
def test_stack_kernel_equals_per_layer_calls(chain, plain_stack, chain_stack):
    # the multi-layer kernel: ids, w, y (and x, r on the chain) bitwise those
    # of one single-layer call per layer, and every layer against the oracle
    layers = chain_stack if chain else plain_stack
    _say("multi-layer kernel, %d layers, chain=%s" % (N_LAYERS, chain))
    ref = _eager(_Run(layers, chain, fused=False))
    run = _Run(layers, chain, fused=True)
    got = _eager(run)
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    worst = _check_stack(run, got)
    _say("  bitwise equal to the per-layer calls; worst max|dy|/max|y| %.2e" % worst)
    # a second call on the same workspace (the epochs continue)
    again = _eager(run)
    for k in ref:
        np.testing.assert_array_equal(again[k], ref[k], err_msg="second call, " + k)


@pytest.mark.parametrize("chain", [False, True], ids=["plain", "chain"])
def test_stack_kernel_graph_replays(chain, plain_stack, chain_stack):
    layers = chain_stack if chain else plain_stack
    run = _Run(layers, chain, fused=True)
    eager = _eager(run)
    graphs = []
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for t in range(N_TOK):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                run.enqueue(t, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        run.y.zero_()
        run.ids.zero_()
        for t in range(N_TOK):
            graphs[t].replay()
            torch.cuda.synchronize()
            # eager single-layer work on the same workspace between replays
            if rep == 1:
                L = layers[0]
                yy = torch.empty(4096, dtype=torch.float32, device="cuda")
                moe.moe_layer_decode(L.dims, L.L, L.x_dev(synth.tokens(5, 0, 1, 4096)), 1, yy,
                                     None, None, run.ws, run.wsb)
        got = run.host()
        for k in eager:
            np.testing.assert_array_equal(got[k], eager[k], err_msg="replay %d, %s" % (rep, k))
    assert moe.moe_get_device_error(run.ws) == 0


def test_stack_kernel_2bit_and_partial_layers():
    # 2-bit codes, and a call over a subset of the layers (3 of 5)
    layers = [gu.DeviceLayer(4096, 1024, 64, 4, bits=2, seed=1007, layer=l) for l in range(5)]
    d = layers[0].dims
    ws = moe.alloc_workspace(d, 1)
    x_h = np.stack([synth.tokens(1007, l, 1, 4096)[0] for l in range(5)])
    x = torch.from_numpy(x_h.view(np.int16)).cuda()
    for sel in (list(range(5)), [1, 2, 4]):
        y = torch.zeros((len(sel), 4096), dtype=torch.float32, device="cuda")
        ids = torch.zeros((len(sel), 4), dtype=torch.int32, device="cuda")
        w = torch.zeros((len(sel), 4), dtype=torch.float32, device="cuda")
        xs = x[sel].contiguous()
        moe.moe_stack_decode(d, [layers[l].L for l in sel], xs, y, ids, w, ws)
        for i, l in enumerate(sel):
            yr = torch.zeros(4096, dtype=torch.float32, device="cuda")
            ir = torch.zeros(4, dtype=torch.int32, device="cuda")
            wr = torch.zeros(4, dtype=torch.float32, device="cuda")
            moe.moe_layer_decode(d, layers[l].L, xs[i], 1, yr, ir, wr, ws)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y[i].cpu().numpy(), yr.cpu().numpy())
            np.testing.assert_array_equal(ids[i].cpu().numpy(), ir.cpu().numpy())
            np.testing.assert_array_equal(w[i].cpu().numpy(), wr.cpu().numpy())
        _oracle_layer_check(layers[sel[-1]], x_h[sel[-1]], ids[-1].cpu().numpy(),
                            w[-1].cpu().numpy(), y[-1].cpu().numpy(), "2-bit layer %d" % sel[-1])
    assert moe.moe_get_device_error(ws) == 0


@pytest.mark.parametrize("chain", [False, True], ids=["plain", "chain"])
def test_stack_kernel_more_layers_than_one_launch(chain):
    # 70 layers (64 per launch): the same layers of 16 experts repeated
    base = [gu.DeviceLayer(4096, 1024, 16, 4, bits=4, seed=1008, layer=l,
                           z_range=synth.workloads.CENTRED_Z) for l in range(5)]
    n = 70
    layers = [base[l % 5] for l in range(n)]
    d = base[0].dims
    ws = moe.alloc_workspace(d, 1)
    ys = []
    for fused in (False, True):
        y = torch.zeros((n, 4096), dtype=torch.float32, device="cuda")
        ids = torch.zeros((n, 4), dtype=torch.int32, device="cuda")
        if chain:
            r = torch.from_numpy(synth.residual(1008, 1, 4096)[0]).cuda()
            xo = torch.zeros((n, 4096), dtype=torch.int16, device="cuda")
            if fused:
                moe.moe_stack_decode_residual(d, [L.L for L in layers], r, xo, y, ids, None, ws)
            else:
                for l, L in enumerate(layers):
                    moe.moe_layer_decode_residual(d, L.L, r, 1, xo[l], y[l], ids[l], None, ws)
            out = (y, ids, r, xo)
        else:
            x = torch.from_numpy(synth.tokens(1008, 0, n, 4096).view(np.int16)).cuda()
            if fused:
                moe.moe_stack_decode(d, [L.L for L in layers], x, y, ids, None, ws)
            else:
                for l, L in enumerate(layers):
                    moe.moe_layer_decode(d, L.L, x[l], 1, y[l], ids[l], None, ws)
            out = (y, ids)
        torch.cuda.synchronize()
        ys.append([o.cpu().numpy() for o in out])
    for a, b in zip(*ys):
        np.testing.assert_array_equal(a, b)
    assert moe.moe_get_device_error(ws) == 0


def test_stack_fallback_dims_run_per_layer_calls():
    # dims the single-token kernel does not cover (H = 1024): the stack entry
    # point runs one single-layer call per layer
    layers = [gu.DeviceLayer(1024, 512, 32, 2, bits=4, seed=1009, layer=l) for l in range(3)]
    d = layers[0].dims
    ws = moe.alloc_workspace(d, 1)
    x_h = synth.tokens(1009, 0, 3, 1024)
    x = torch.from_numpy(x_h.view(np.int16)).cuda()
    y = torch.zeros((3, 1024), dtype=torch.float32, device="cuda")
    ids = torch.zeros((3, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((3, 2), dtype=torch.float32, device="cuda")
    moe.moe_stack_decode(d, [L.L for L in layers], x, y, ids, w, ws)
    torch.cuda.synchronize()
    for l, L in enumerate(layers):
        _oracle_layer_check(L, x_h[l], ids[l].cpu().numpy(), w[l].cpu().numpy(),
                            y[l].cpu().numpy(), "fallback layer %d" % l)


@pytest.mark.parametrize("chain", [False, True], ids=["plain", "chain"])
def test_stack_layers_against_oracle(chain, plain_stack, chain_stack):
    layers = chain_stack if chain else plain_stack
    _say("stack of %d layers, chain=%s" % (N_LAYERS, chain))
    run = _Run(layers, chain)
    sp = torch.cuda.current_stream().cuda_stream
    for t in range(N_TOK):
        run.enqueue(t, sp)
    torch.cuda.synchronize()
    assert moe.moe_get_device_error(run.ws) == 0
    eager = run.host()
    worst = _check_stack(run, eager)
    _say("  worst max|dy|/max|y| over %d layers x %d tokens: %.2e" % (N_LAYERS, N_TOK, worst))
    # the same tokens replayed from captured graphs, twice, with eager work
    # between the replays: bitwise equal to the eager run
    graphs = []
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for t in range(N_TOK):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                run.enqueue(t, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(2):
        run.y.zero_()
        run.ids.zero_()
        for t in range(N_TOK):
            graphs[t].replay()
            torch.cuda.synchronize()
        got = run.host()
        for k in ("y", "ids", "w", "x"):
            np.testing.assert_array_equal(got[k], eager[k], err_msg="replay %d, %s" % (rep, k))
    assert moe.moe_get_device_error(run.ws) == 0
