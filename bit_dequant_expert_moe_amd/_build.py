"""Builds libmoe.so (the C-ABI library) in-tree with hipcc for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = [os.path.join(CSRC, "moe_host.cpp"), os.path.join(CSRC, "moe_kernels.hip"),
           os.path.join(CSRC, "moe_fused.hip"), os.path.join(CSRC, "moe_grouped.hip"),
           os.path.join(CSRC, "moe_tier.cpp"), os.path.join(CSRC, "moe_probe.hip"),
           os.path.join(CSRC, "moe_stack.hip"), os.path.join(CSRC, "moe_noalloc.hip"),
           os.path.join(CSRC, "moe_timing.cpp")]
HEADERS = [os.path.join(CSRC, "moe_internal.h"), os.path.join(CSRC, "moe_device.h"),
           os.path.join(CSRC, "moe_fused_dev.h"),
           os.path.join(os.path.dirname(HERE), "include", "moe.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-function",
         # no packed-FP32 instructions in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core results in ordinary VGPRs: with accumulation registers
         # the grouped GEMM needs 288 registers per lane (one wave per SIMD)
         # and reads every result back with v_accvgpr_read
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def build(force: bool = True, extra=None, out=None) -> str:
    """Builds libmoe.so, or `out` with the extra hipcc flags `extra`."""
    dst = out or LIB
    srcs = SOURCES + HEADERS
    if not force and os.path.exists(dst) and all(
            os.path.getmtime(s) <= os.path.getmtime(dst) for s in srcs):
        return dst
    tmp = dst + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(extra or []), "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    print(build())
