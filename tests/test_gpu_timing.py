"""Per-stage timing (moe_timing_set / moe_timing_read) on the GPU: the
stages each path runs are counted once per call, their times are positive
and add up to no more than the call's own duration, and calls captured into
a graph record nothing."""
import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_dequant_expert_moe_amd as moe  # noqa: E402


@pytest.fixture(scope="module")
def layer():
    # 16 experts of the full shape: the single-token and multi-layer kernels
    # cover it, T >= 2 takes the grouped path
    return gu.DeviceLayer(4096, 1024, 16, 4, bits=4, seed=1200)


def test_stage_timing(layer):
    L = layer
    H = L.dims.hidden
    moe.moe_timing_set(True)
    try:
        moe.moe_timing_read(reset=True)
        T = 8
        x = L.x_dev(synth.tokens(1200, 0, T, H))
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, 4), dtype=torch.int32, device="cuda")
        ws = moe.alloc_workspace(L.dims, T)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        moe.moe_layer_decode(L.dims, L.L, x, T, y, ids, None, ws)
        e1.record()
        torch.cuda.synchronize()
        wall = e0.elapsed_time(e1)
        t = moe.moe_timing_read(reset=True)
        assert set(t) == {"route", "bucket", "gateup", "down", "combine"}, t
        assert all(n == 1 and ms > 0 for ms, n in t.values()), t
        total = sum(ms for ms, _ in t.values())
        assert total <= wall * 1.05 + 0.005, (total, wall)

        # one token: the single-token kernel, one stage per call
        for _ in range(3):
            moe.moe_layer_decode(L.dims, L.L, x[:1], 1, y[:1], ids[:1], None, ws)
        t = moe.moe_timing_read(reset=True)
        assert set(t) == {"layer"} and t["layer"][1] == 3, t

        # two layers of one token in one multi-layer launch
        arr = moe.layer_array([L.L, L.L])
        moe.moe_stack_decode(L.dims, arr, x[:2], y[:2], ids[:2], None, ws)
        t = moe.moe_timing_read(reset=False)
        assert set(t) == {"stack"} and t["stack"][1] == 1 and t["stack"][0] > 0, t
        # without reset the totals stay; with it they start again
        assert moe.moe_timing_read(reset=True) == t
        assert moe.moe_timing_read() == {}

        # calls captured into a graph record nothing, nor do their replays
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                moe.moe_layer_decode(L.dims, L.L, x, T, y, ids, None, ws,
                                     stream=torch.cuda.current_stream().cuda_stream)
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        assert moe.moe_timing_read() == {}

        # switched off: nothing is recorded
        moe.moe_timing_set(False)
        moe.moe_layer_decode(L.dims, L.L, x, T, y, ids, None, ws)
        torch.cuda.synchronize()
        assert moe.moe_timing_read() == {}
    finally:
        moe.moe_timing_set(False)
        moe.moe_timing_read(reset=True)
