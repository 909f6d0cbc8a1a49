"""Run by tests/test_gpu_paths.py in a child process whose environment
selects a dispatch path (MOE_DISABLE_FUSED=1: the three-kernel single-token
path, and the grouped path from two tokens on; MOE_DISABLE_GROUPED=1: the
per-token kernels for more tokens than the single-token kernel takes one
launch each).  The library reads these switches once per process, hence the
child.  Prints one JSON line with the worst relative output error against the
oracle."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


def main():
    worst, cases = 0.0, 0
    for bits in (4, 2):
        L = gu.DeviceLayer(4096, 1024, 32, 4, bits=bits, seed=3000 + bits)
        for T in (1, 2, 5):
            x = synth.tokens(3000 + bits, T, T, 4096)
            out = L.decode(x, want_logits=True)
            assert out["err"] == 0
            _, _, logits_o, gap_o = oracle.route(L.od, L.router_h, x)
            gu.check_routing(L.od, out["ids"], out["w"], logits_o, gap_o, 4)
            wf = np.empty((T, 4))
            for t in range(T):
                sel = logits_o[t][out["ids"][t]]
                e = np.exp(sel - sel.max())
                wf[t] = e / e.sum()
            y_o = oracle.expert_forward(L.od, L.blob_host, L.shared_host(), x, out["ids"], wf)
            worst = max(worst, gu.max_rel_err(out["y"], y_o))
            cases += 1
        # the residual entry point on the same path
        r = synth.residual(3000 + bits, 2, 4096)
        o = L.decode_residual(r)
        assert o["err"] == 0
        for t in range(2):
            gu.check_norm(o["x"][t], r[t])
            np.testing.assert_array_equal(o["r"][t], (r[t] + o["y"][t]).astype(np.float32))
        cases += 1
    print(json.dumps({"worst_rel_err": worst, "cases": cases}), flush=True)


if __name__ == "__main__":
    main()
