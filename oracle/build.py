"""Build the CPU oracle (plain C) into ``oracle/libqr_oracle.so``.

Test infrastructure only: see ``oracle/__init__.py``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qr_oracle.c")
LIB = os.path.join(HERE, "libqr_oracle.so")

# Plain IEEE binary32 semantics: no fast-math, no FMA contraction.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(src=SRC, out=LIB, cc="gcc", quiet=True, extra=()):
    """Compile ``src`` into the shared library ``out`` (``extra``: more compiler
    flags, e.g. sanitizers); returns ``out``."""
    cmd = [cc, *CFLAGS, *extra, "-o", out, src, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{res.stderr}")
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
