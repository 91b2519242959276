"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; CPU only).

qr_api.hip is compiled with the sanitizers on its host side and linked with
stand-ins for the launch functions of the other translation units
(tests/c_abi/launch_stubs.cpp); tests/c_abi/validate_check.c then drives every
rejection path of include/qr.h (n == 0 among them) and a set of accepted calls,
which end in a stand-in instead of a launch.  No GPU work runs."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
INC = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_quantized_all_amd", "csrc")]
# host side only: every sanitizer flag goes to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, (" ".join(cmd), r.stderr[-3000:])
    return r


@pytest.mark.timeout(600)
def test_c_abi_checks_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers are not installed")
    d = str(tmp_path)
    common = ["-x", "hip", "-std=c++17", "-O0", "-g", "-fPIC", *INC, *HOST_SAN]
    # the device side keeps the library's optimization level: the kernels'
    # buffer resources must stay in scalar registers, which -O0 does not do
    _run([HIPCC, "--offload-arch=gfx950", *common, "-Xarch_device", "-O3", "-c",
          os.path.join(ROOT, "bit_quantized_all_amd", "csrc", "qr_api.hip"), "-o", "api.o"], d)
    _run([HIPCC, "--cuda-host-only", *common, "-c",
          os.path.join(ROOT, "tests", "c_abi", "launch_stubs.cpp"), "-o", "stubs.o"], d)
    _run([CLANG + "++", "-shared", *LINK_SAN, "api.o", "stubs.o", "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", "-o", "libqr_hostsan.so"], d)
    _run([CLANG, "-std=c11", "-Wall", "-Werror", "-g", *LINK_SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "c_abi", "validate_check.c"), "-L", d, "-lqr_hostsan",
          "-Wl,-rpath," + d, "-o", "validate_check"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([os.path.join(d, "validate_check")], cwd=d, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "all checks passed" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
