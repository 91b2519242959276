"""Build the HIP library ``bit_quantized_all_amd/libqr.so`` for gfx950.

Cross-compiles with hipcc (no GPU needed).  Floating-point contraction is off
so that every rounding in the codec happens where the source writes it
(explicit fmaf calls only where a fused result is exact), and packed fp32
instructions are disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "qr_kernels.hip")
LIB = os.path.join(HERE, "libqr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def build(out=LIB, extra=(), quiet=True, src=SRC):
    """Compile the kernels and the C ABI into ``out``; returns ``out``."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"HIP build failed: {' '.join(cmd)}\n{res.stderr}")
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


TEST_HELPER_SRC = os.path.join(ROOT, "tests", "gpu_helpers", "scale_check.hip")
TEST_HELPER_LIB = os.path.join(ROOT, "tests", "gpu_helpers", "libscale_check.so")


def build_test_helpers(quiet=True):
    """Test-only HIP helper that exercises the codec's device functions directly."""
    return build(out=TEST_HELPER_LIB, src=TEST_HELPER_SRC, quiet=quiet)


if __name__ == "__main__":
    print(build(quiet=False))
