"""The benchmark's command line, the parts that need no GPU: the options it
documents, and the refusal of more than one GPU (this library has no
multi-GPU path)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_help_lists_the_options():
    r = _run("--help")
    assert r.returncode == 0, r.stderr
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--timing", "--layer-trace",
                "--no-cpu-baseline", "--calib-copy"):
        assert opt in r.stdout, opt
    for wl in ("stack60", "stack60_chain", "stack60_2bit", "layer", "batch64", "prefill4096",
               "stack8_tier"):
        assert wl in r.stdout, wl


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line
