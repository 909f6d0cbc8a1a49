"""The dispatch paths that the default process never takes for the main
shape (hidden 4096, intermediate 1024, top-4): the three-kernel single-token
path, the grouped path for two tokens and the per-token kernels for several
tokens.  Each runs in a child process (tests/path_check.py) with its switch
set, against the oracle."""
import json
import os
import subprocess
import sys

import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("switch", ["MOE_DISABLE_FUSED", "MOE_DISABLE_GROUPED"])
def test_path_against_oracle(switch):
    env = dict(os.environ)
    env[switch] = "1"
    print("path check with", switch, flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "path_check.py")], env=env,
                       capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print("  ", res, flush=True)
    assert res["cases"] == 8
    assert res["worst_rel_err"] <= gu.Y_TOL
