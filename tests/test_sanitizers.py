"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU only).

Two sanitized builds, each exercised by the CPU tests that reach it, in a
child process of its own (the two sanitizer runtimes cannot share a process):

* the oracle (``oracle.c``, gcc ``-fsanitize=address,undefined``) under
  ``tests/test_oracle.py``;
* the C-ABI library's host code (argument validation, layouts, workspace
  sizing and the tier planner in ``moe_host.cpp`` / ``moe_tier.cpp``; hipcc
  with the sanitizers on the host pass only, device code as usual) under
  ``tests/test_abi.py`` and ``tests/test_tier.py``.

Every UB check halts (``halt_on_error`` / ``-fno-sanitize-recover``), so any
report fails the child's exit status; the report text is checked as well.
Leak checking is off: the Python interpreter itself keeps memory until exit.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CLANG_RT = "/opt/rocm/llvm/lib/clang"

# checks, in the child, that the sanitized library is the one loaded, then
# runs the given test files
_CHILD = r"""
import sys, pytest
{load}
maps = open('/proc/self/maps').read()
assert {path!r} in maps, 'sanitized library not loaded'
sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu', *sys.argv[1:]]))
"""


def _run(env_extra, load, path, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", _CHILD.format(load=load, path=path), *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out, out[-6000:]
    assert "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out, out[-2000:]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    if not os.path.isdir(CLANG_RT):
        return None
    for v in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liboracle_san.so")
    oracle.build(out=lib, extra=["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                                 "-fno-sanitize-recover=all"])
    _run({"MOE_ORACLE_LIB": lib, "LD_PRELOAD": asan + " " + ubsan},
         "import oracle; oracle.lib()", lib, ["tests/test_oracle.py"])


def test_host_library_under_asan_ubsan(tmp_path):
    from bit_dequant_expert_moe_amd import _build
    asan = _clang_asan()
    if asan is None or not os.path.exists(_build.HIPCC):
        pytest.skip("hipcc or its AddressSanitizer runtime not installed")
    lib = str(tmp_path / "libmoe_san.so")
    _build.build(out=lib, extra=["-Xarch_host", "-fsanitize=address",
                                 "-Xarch_host", "-fsanitize=undefined",
                                 "-Xarch_host", "-fno-sanitize-recover=all",
                                 "-Xarch_host", "-fno-omit-frame-pointer"])
    _run({"MOE_LIB": lib, "LD_PRELOAD": asan},
         "import bit_dequant_expert_moe_amd as m; m.lib()", lib,
         ["tests/test_abi.py", "tests/test_tier.py"])
