"""The C ABI from plain C99: tests/c/abi_c.c is compiled with gcc against
include/moe.h and libmoe.so (the header must be valid C) and run: host-only
calls on the CPU, and one layer on all-zero weights on the GPU (closed-form
result: ids 0 .. K-1, weights 1/K, y = 0) through the three-kernel path
(T = 1 at these dims) and the grouped path (T = 4), and two layers in the
multi-layer kernel, plain and chained through the residual with the entry
point that takes no workspace (the residual comes back unchanged)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bit_dequant_expert_moe_amd")
SRC = os.path.join(ROOT, "tests", "c", "abi_c.c")
ROCM = "/opt/rocm"


def _compile(out, gpu):
    lib = os.path.join(LIBDIR, "libmoe.so")
    if not os.path.exists(lib):
        pytest.skip("libmoe.so is not built")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I" + os.path.join(ROOT, "include"), SRC, "-o", out, lib,
           "-Wl,-rpath," + LIBDIR]
    if gpu:
        # (the HIP runtime's own headers are not -pedantic clean)
        cmd.remove("-pedantic")
        cmd[1:1] = ["-DMOE_C_GPU", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]
        cmd += ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_c_header_and_host_calls(tmp_path):
    exe = str(tmp_path / "abi_c")
    _compile(exe, gpu=False)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.gpu
def test_c_layer_decode_on_zero_weights(tmp_path):
    exe = str(tmp_path / "abi_c_gpu")
    _compile(exe, gpu=True)
    r = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
