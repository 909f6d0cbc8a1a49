"""The no-allocation multi-layer residual decode against the same call with a
caller workspace: x, y, ids, w and the residual must be bitwise equal, on
calls in a row of decreasing size, on dims the multi-layer kernel covers and
on dims it does not (per-layer path), and when the call is captured in a graph
and replayed (after a first, uncaptured call has set the array up)."""
import numpy as np
import pytest

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
def big():
    # the decode dims: one launch of the multi-layer kernel per call
    return [gu.DeviceLayer(4096, 1024, 512, 4, bits=4, seed=1002, layer=l,
                           z_range=synth.workloads.CENTRED_Z) for l in range(4)]


@pytest.fixture(scope="module")
def small():
    # dims the multi-layer kernel does not cover: one layer call after another
    return [gu.DeviceLayer(512, 256, 16, 2, bits=4, seed=1003, layer=l) for l in range(3)]


class _Bufs:
    def __init__(self, d, n, seed):
        H, K = d.hidden, d.top_k
        self.r0 = torch.from_numpy(synth.residual(seed, 1, H, 0.97)[0].copy()).cuda()
        self.r = self.r0.clone()
        self.x = torch.full((n, H), -1, dtype=torch.int16, device="cuda")
        self.y = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
        self.ids = torch.full((n, K), -1, dtype=torch.int32, device="cuda")
        self.w = torch.full((n, K), float("nan"), dtype=torch.float32, device="cuda")

    def host(self):
        return [t.cpu().numpy().view(np.uint8) for t in (self.r, self.x, self.y, self.ids, self.w)]


def _with_ws(layers, n, seed):
    d = layers[0].dims
    arr = moe.layer_array([L.L for L in layers[:n]])
    b = _Bufs(d, n, seed)
    ws = moe.alloc_workspace(d, 1)
    moe.moe_stack_decode_residual(d, arr, b.r, b.x, b.y, b.ids, b.w, ws, ws.numel())
    torch.cuda.synchronize()
    return b.host()


def _same(a, b, label):
    names = ("resid", "x", "y", "ids", "w")
    for name, u, v in zip(names, a, b):
        assert np.array_equal(u, v), "%s: %s differs" % (label, name)
    _say("  %s: bitwise equal" % label)


def _noalloc(layers, n, seed):
    d = layers[0].dims
    arr = moe.layer_array([L.L for L in layers[:n]])
    b = _Bufs(d, n, seed)
    moe.moe_stack_decode_residual_noalloc(d, arr, b.r, b.x, b.y, b.ids, b.w)
    torch.cuda.synchronize()
    return b.host()


def test_noalloc_equals_workspace_calls(big, small):
    for layers, n, seed, label in [(big, 4, 11, "4 layers, 4096 x 1024"),
                                   (big, 2, 12, "2 layers, 4096 x 1024"),
                                   (small, 3, 13, "3 layers, 512 x 256 (per-layer path)"),
                                   (small, 1, 14, "1 layer, 512 x 256 (per-layer path)"),
                                   (big, 3, 15, "3 layers, 4096 x 1024 after the per-layer path")]:
        _say("case:", label)
        _same(_with_ws(layers, n, seed), _noalloc(layers, n, seed), label)


def test_noalloc_graph_replays(big):
    d = big[0].dims
    n = 3
    arr = moe.layer_array([L.L for L in big[:n]])
    want = _with_ws(big, n, 21)
    # eager first call (sets the array up if no test before this one did)
    first = _noalloc(big, n, 21)
    _same(want, first, "eager")
    b = _Bufs(d, n, 21)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            moe.moe_stack_decode_residual_noalloc(d, arr, b.r, b.x, b.y, b.ids, b.w,
                                                  stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        b.r.copy_(b.r0)
        b.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, b.host(), "graph replay %d" % rep)
        # eager work between replays: the same call with a workspace
        _same(want, _with_ws(big, n, 21), "eager call after replay %d" % rep)
