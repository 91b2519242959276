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
_CSRC = os.path.join(HERE, "csrc")
# (source, extra flags): the mixed-format and asymmetric reduces are built once
# per input format
SOURCES = [(os.path.join(_CSRC, "qr_api.hip"), [])] + [
    (os.path.join(_CSRC, "qr_reduce_mixed.hip"), [f"-DQR_MIXED_IN={b}"]) for b in (3, 4, 8)] + [
    (os.path.join(_CSRC, "qr_asym.hip"), [f"-DQR_ASYM_IN={f}"]) for f in (20, 24)] + [
    (os.path.join(_CSRC, "qr_fp4.hip"), [])]
LIB = os.path.join(HERE, "libqr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def _run(cmd):
    return subprocess.run(cmd, capture_output=True, text=True)


def build(out=LIB, extra=(), quiet=True, sources=None):
    """Compile the translation units in parallel and link them into ``out``."""
    import concurrent.futures
    import tempfile

    sources = SOURCES if sources is None else sources
    with tempfile.TemporaryDirectory() as tmpdir:
        sources = [s if isinstance(s, tuple) else (s, []) for s in sources]
        objs = [os.path.join(tmpdir, f"{i}_{os.path.basename(src)}.o") for i, (src, _) in enumerate(sources)]
        cmds = [[HIPCC, *FLAGS, *extra, *defs, "-c", "-o", obj, src]
                for (src, defs), obj in zip(sources, objs)]
        with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, res in zip(cmds, results):
            if res.returncode != 0:
                raise RuntimeError(f"HIP build failed: {' '.join(cmd)}\n{res.stderr}")
            if not quiet and res.stderr:
                sys.stderr.write(res.stderr)
        tmp = out + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        res = _run(link)
        if res.returncode != 0:
            raise RuntimeError(f"HIP link failed: {' '.join(link)}\n{res.stderr}")
        os.replace(tmp, out)
    return out


TEST_HELPER_SRCS = [os.path.join(ROOT, "tests", "gpu_helpers", f) for f in ("scale_check.hip", "fp4_check.hip", "asym_check.hip")]
TEST_HELPER_LIB = os.path.join(ROOT, "tests", "gpu_helpers", "libscale_check.so")


SMALL_GRID_LIB = os.path.join(ROOT, "tests", "gpu_helpers", "libqr_smallgrid.so")
ABI_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
ABI_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_abi_check():
    """A plain C program (gcc, no C++) that calls the C ABI of include/qr.h
    against libqr.so, found through an rpath relative to the binary."""
    cmd = ["gcc", "-std=c11", "-Wall", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-o", ABI_CHECK_BIN, ABI_CHECK_SRC,
           "-L", HERE, "-lqr", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../bit_quantized_all_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = _run(cmd)
    if res.returncode != 0:
        raise RuntimeError(f"C ABI check build failed: {' '.join(cmd)}\n{res.stderr}")
    return ABI_CHECK_BIN


def build_test_helpers(quiet=True):
    """Test-only HIP libraries: a helper that exercises the codec's device
    functions directly, and the library itself built with its grid capped at 3
    workgroups, so that every kernel's grid-stride loop (and the encode's
    prefetch of the next tile) runs at small sizes."""
    build(out=SMALL_GRID_LIB, extra=["-DQR_MAX_GROUPS=3"], quiet=quiet)
    build_abi_check()
    return build(out=TEST_HELPER_LIB, sources=TEST_HELPER_SRCS, quiet=quiet)


def main(argv=None):
    """python -m bit_quantized_all_amd.build [--out PATH] [-DNAME=VALUE ...]:
    build the library (by default in place); definitions select the
    compile-time variants of the kernels (the macros of csrc/qr_kernels.hpp
    and csrc/qr_codec.hpp), e.g. for a measurement of a variant next to the
    default build (bench.py --lib PATH)."""
    import argparse
    ap = argparse.ArgumentParser(description=main.__doc__)
    ap.add_argument("--out", default=LIB)
    args, defs = ap.parse_known_args(argv)
    bad = [d for d in defs if not d.startswith("-D")]
    if bad:
        ap.error(f"unexpected arguments {bad} (only -DNAME=VALUE definitions)")
    print(build(out=os.path.abspath(args.out), extra=defs, quiet=False))


if __name__ == "__main__":
    main()
