"""The oracle's pins and the model cross-check, run against a build of the
oracle with gcc's AddressSanitizer and UndefinedBehaviorSanitizer (including
float-to-integer conversion overflow), so that an out-of-bounds access, an
uninitialized tile region or an undefined conversion in the oracle fails the
suite instead of passing by luck.  CPU only."""
import os
import subprocess
import sys

import pytest

import oracle.build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
SANITIZE = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-g"]

SCRIPT = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle, oracle_pins as P, test_oracle_model as T
o = oracle.Oracle(sys.argv[1])
for pin in P.ALL_PINS:
    pin(o)
for fmt in T.FORMATS:
    for dtype in P.DTYPES:
        T.test_encode_decode_match_model(o, fmt, dtype)
        T.test_reduce_matches_model(o, fmt, dtype)
for fmt_in, fmt_out in T.MIXED:
    T.test_mixed_reduce_matches_model(o, fmt_in, fmt_out)
T.test_fp16_sum_overflow_matches_model(o)
print("sanitized oracle: all checks passed", flush=True)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = obuild.build(out=str(tmp_path / "libqr_oracle_san.so"), extra=SANITIZE)
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", SCRIPT, lib, HERE, os.path.dirname(HERE)],
                       env=env, capture_output=True, text=True, timeout=850)
    assert r.returncode == 0 and "all checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-6000:])
