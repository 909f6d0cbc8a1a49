"""GPU checks of the off-HBM expert tier through the C ABI: experts in pinned
host memory, a few device slots (so that calls evict), every output bitwise
equal to moe_route + moe_expert_forward over the same experts held in device
memory, and sampled calls against the float64 oracle (routing exact away
from near-ties, y within 2e-3 max|y|, teacher-forced on the tier's routing)."""
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


def _aligned(n, device, align=256, pin=False):
    if device == "cpu":
        t = torch.empty(n + align, dtype=torch.uint8, pin_memory=pin)
    else:
        t = torch.empty(n + align, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % align
    return t[off:off + n]


def _setup(bits, n_layers, n_slots, t_max, E=64):
    layers = [gu.DeviceLayer(4096, 1024, E, 4, bits=bits, seed=2000 + bits, layer=l)
              for l in range(n_layers)]
    d = layers[0].dims
    blob = moe.moe_expert_bytes(d)
    host = []
    for L in layers:
        h = _aligned(E * blob, "cpu", pin=True)
        h.copy_(L.experts[:E * blob].cpu())
        host.append(h)
    slots = _aligned(n_slots * blob, "cuda")
    staging = _aligned(moe.moe_tier_staging_bytes(d, t_max), "cpu", pin=True)
    scratch = _aligned(moe.moe_tier_device_bytes(d, t_max), "cuda")
    copy_stream = torch.cuda.Stream()
    tier = moe.Tier(d, [h.data_ptr() for h in host], blob, slots, blob, n_slots, staging,
                    scratch, t_max=t_max, copy_stream=copy_stream)
    return layers, host, tier, (slots, staging, scratch, copy_stream)


@pytest.mark.parametrize("bits,T,n_slots", [(4, 1, 4), (4, 1, 14), (2, 1, 16), (4, 3, 40)])
def test_tier_equals_resident(bits, T, n_slots):
    _say("tier bits %d T %d slots %d" % (bits, T, n_slots))
    layers, host, tier, keep = _setup(bits, 3, n_slots, T)
    d = layers[0].dims
    blob_b = moe.moe_expert_bytes(d)
    wsb = moe.moe_tier_workspace_bytes(d, n_slots, T)
    ws = _aligned(wsb, "cuda")
    moe.moe_workspace_init(ws, wsb)
    ws_ref = moe.alloc_workspace(d, T)
    ntok = 6
    x_all = synth.tokens_ar1(2100 + bits, 0, ntok * T, 4096, 0.9)
    n_valid = 0
    for t in range(ntok):
        for l, L in enumerate(layers):
            x = L.x_dev(x_all[t * T:(t + 1) * T])
            y = torch.empty((T, 4096), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, 4), dtype=torch.int32, device="cuda")
            w = torch.empty((T, 4), dtype=torch.float32, device="cuda")
            tier.decode(l, L.router, L.shared, x, T, y, ids, w, ws, wsb)
            y_r = torch.empty_like(y)
            ids_r = torch.empty_like(ids)
            w_r = torch.empty_like(w)
            moe.moe_route(d, L.router, x, T, ids_r, w_r, None, ws_ref)
            moe.moe_expert_forward(d, L.L, x, T, ids_r, w_r, y_r, ws_ref)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(ids.cpu().numpy(), ids_r.cpu().numpy())
            np.testing.assert_array_equal(w.cpu().numpy(), w_r.cpu().numpy())
            np.testing.assert_array_equal(y.cpu().numpy(), y_r.cpu().numpy())
            n_valid += len({(int(e)) for e in ids.cpu().numpy().reshape(-1)})
            if t in (1, ntok - 1):
                # the oracle on the bytes the tier copied from host memory:
                # routing from x, y teacher-forced on the tier's choice
                xh = x_all[t * T:(t + 1) * T]
                ids_h, w_h, y_h = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
                _, _, logits_o, gap_o = oracle.route(L.od, L.router_h, xh)
                gu.check_routing(L.od, ids_h, w_h, logits_o, gap_o, 4)
                wf = np.empty((T, 4))
                for tt in range(T):
                    sel = logits_o[tt][ids_h[tt]]
                    wf[tt] = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
                blob_of = (lambda e, l=l: host[l][e * blob_b:(e + 1) * blob_b].numpy())
                y_o = oracle.expert_forward(L.od, blob_of, L.shared_host(), xh, ids_h, wf)
                err = gu.max_rel_err(y_h, y_o)
                _say("  token %d layer %d: max|dy|/max|y| = %.2e (oracle)" % (t, l, err))
                assert err <= gu.Y_TOL
    assert moe.moe_get_device_error(ws) == 0
    st = tier.stats()
    _say("  stats", st)
    assert st["hits"] + st["misses"] == n_valid
    assert st["bytes"] == st["misses"] * moe.moe_expert_bytes(d)
    assert st["evictions"] > 0
    if n_slots > 3 * T * 4:  # room for reuse across tokens once every layer is cached
        assert st["hits"] > 0
    tier.close()
