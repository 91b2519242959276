"""Checks of the gfx950 machine code in the built ``libqr.so`` (CPU only).

The code objects are extracted from the library's offload bundle with
``llvm-objdump --offloading``; their kernel metadata and their disassembly are
read with the ROCm LLVM tools.  What is checked:

- no kernel uses scratch memory or spills registers (a spill would turn the
  streaming kernels into scratch traffic);
- no packed fp32 instruction appears: the library is built with the
  ``packed-fp32-ops`` target feature turned off, and this shows the flag took
  effect in every translation unit;
- no round-toward-zero conversion to fp16 appears: every conversion to the
  I/O dtype must round to nearest even, as the codec defines it;
- every format and dtype has its encode, decode and reduce kernels.
"""
import functools
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_quantized_all_amd", "libqr.so")
LLVM = "/opt/rocm/llvm/bin"
OBJDUMP = os.path.join(LLVM, "llvm-objdump")
READELF = os.path.join(LLVM, "llvm-readelf")

FORMATS = (3, 4, 8, 20, 24, 36)


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    if not (os.path.exists(OBJDUMP) and os.path.exists(READELF)):
        pytest.skip("ROCm LLVM tools are not installed")
    if not os.path.exists(LIB):
        pytest.skip("libqr.so is not built")
    d = tmp_path_factory.mktemp("isa")
    lib = str(d / "libqr.so")
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
    objs = sorted(str(p) for p in d.iterdir() if p.name.endswith("gfx950"))
    assert objs, "no gfx950 code object in libqr.so"
    return objs


@functools.lru_cache(maxsize=None)
def _kernels(obj):
    """{kernel name: metadata} from the code object's AMDGPU metadata note (YAML)."""
    import yaml

    text = subprocess.run([READELF, "--notes", obj], check=True, capture_output=True, text=True).stdout
    start = text.index("amdhsa.kernels:")
    end = text.find("\n...", start)
    loader = getattr(yaml, "CSafeLoader", yaml.SafeLoader)   # the C parser when present
    md = yaml.load(text[start:end if end >= 0 else None], Loader=loader)
    return {k[".name"]: k for k in md["amdhsa.kernels"]}


def test_no_scratch_and_no_spills(code_objects):
    seen = 0
    for obj in code_objects:
        for name, md in _kernels(obj).items():
            seen += 1
            assert md[".private_segment_fixed_size"] == 0, name
            assert md[".vgpr_spill_count"] == 0 and md[".sgpr_spill_count"] == 0, name
            assert md[".vgpr_count"] <= 256, name
    assert seen > 0


def test_every_format_has_its_kernels(code_objects):
    names = set()
    for obj in code_objects:
        names |= set(_kernels(obj))
    for fmt in FORMATS:
        for dt in (0, 1):
            for kind in ("encode_kernel", "decode_kernel"):
                want = f"{kind}ILi{fmt}ELi{dt}E"
                assert any(want in n for n in names), want
        assert any(f"reduce_kernelILi{fmt}E" in n for n in names), fmt


def test_no_packed_fp32_and_no_truncating_conversions(code_objects):
    bad = re.compile(r"\b(v_pk_(?:add|mul|fma)_f32|v_cvt_pkrtz\w*|scratch_\w+)\b")
    for obj in code_objects:
        asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", obj], check=True, capture_output=True,
                             text=True).stdout
        assert "v_cvt_f32_f16" in asm or "v_cvt_pk_f16_f32" in asm or "v_cvt_pk_bf16_f32" in asm, obj
        hits = sorted(set(bad.findall(asm)))
        assert not hits, (os.path.basename(obj), hits)
