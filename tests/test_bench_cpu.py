"""Host logic of bench.py (CPU only): algorithmic bytes, the tile sizes it
assumes, the counter ingestion and its calibration, the kernel-source guard
on stored traffic, and the single-GPU exit."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_algorithmic_bytes_of_the_bench_workload():
    """[32 x 1024 x 4096] fp16 per rank, INT4 (1152 B per 2048 values), R = 8:
    encode 2 + c bytes per value, reduce R*c + c + 2."""
    w = W.WORKLOADS["int4_r8_fp16_32x1024x4096"]
    n = 32 * 1024 * 4096
    ab = bench.algorithmic_bytes(w)
    assert ab["encode"] == n * 2 + n // 2048 * 1152 == 343_932_928
    assert ab["reduce"] == 8 * (n // 2048 * 1152) + n // 2048 * 1152 + 2 * n == 947_912_704
    assert ab["decode"] == ab["encode"]


def test_mixed_output_format_bytes():
    w = W.WORKLOADS["int6_r8_fp16_32x1024x4096"]      # INT4 inputs, INT8 re-encoded sum
    tiles = w.n // 2048
    assert bench.algorithmic_bytes(w)["reduce"] == 8 * tiles * 1152 + tiles * 2176 + 2 * w.n


def test_tile_sizes_match_the_library_and_the_oracle():
    import bit_quantized_all_amd as qa
    import oracle

    o = oracle.default()
    for fmt, tb in bench.TILE_BYTES.items():
        fid = bench.FORMAT_IDS[fmt]
        assert qa.qr_packed_bytes(fmt, 2048) == tb == o.packed_bytes(fid, 2048), fmt


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_ingest_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE are scaled so that the copy of one rank's input
    (n * 2 bytes each way) reads as its known size; torch's own reduce kernel and
    other kernels are ignored; medians over dispatches."""
    wl = "int4_r8_fp16_32x1024x4096"
    w = W.WORKLOADS[wl]
    ab = bench.algorithmic_bytes(w)
    kib = w.n * 2 / 1024
    enc_r, enc_w = w.n * 2 / 1024, (ab["encode"] - w.n * 2) / 1024
    red_r, red_w = (ab["reduce"] - ab["encode"]) / 1024, ab["encode"] / 1024
    fetch = [("copy_kernel<...>", kib / 2), ("copy_kernel<...>", kib / 2),
             ("void qr::encode_kernel<4, 0>(...)", enc_r / 2), ("void qr::encode_kernel<4, 0>(...)", enc_r / 2 + 1),
             ("void qr::encode_kernel<4, 0>(...)", enc_r / 2 - 1),
             ("void qr::reduce_kernel<4, 4, 0, 8, true>(qr::ReduceArgs)", red_r / 2),
             ("void at::native::reduce_kernel<512, 1>(...)", 99.0), ("distribution_kernel", 5.0)]
    write = [("copy_kernel<...>", kib), ("void qr::encode_kernel<4, 0>(...)", enc_w),
             ("void qr::reduce_kernel<4, 4, 0, 8, true>(qr::ReduceArgs)", red_w)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out_json = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out_json))
    bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), wl)
    d = json.load(open(out_json))[wl]
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["bytes_per_launch"]["encode"] == pytest.approx(ab["encode"], rel=1e-9)
    assert d["bytes_per_launch"]["reduce"] == pytest.approx(ab["reduce"], rel=1e-9)
    assert d["kernel_source_hash"] == bench.kernel_source_hash()


def test_stored_traffic_needs_the_same_kernel_sources(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"wl": {"kernel_source_hash": "abc", "bytes_per_launch": {"encode": 7}}}))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(p))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.traffic_from_profiles("encode", "wl") == 7
    assert bench.traffic_from_profiles("reduce", "wl") is None
    assert bench.traffic_from_profiles("encode", "other") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.traffic_from_profiles("encode", "wl") is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_buffer_sets_cover_every_kernels_reads_and_writes():
    """The rotation is sized by the smallest per-kernel read or write footprint
    of a set, so that no kernel re-reads its inputs from the last-level cache
    and no kernel re-writes an output that may still be dirty there."""
    import workloads as W
    mib = 1 << 20
    wb = W.WORKLOADS["int4_r8_fp16_32x1024x4096"]          # reduce writes 72 + 256 MiB per set
    assert bench.buffer_sets(wb, 1152 * wb.n // 2048, 512) == 2
    wc = W.WORKLOADS["int4_fp16_codec_32x1024x4096"]       # decode reads, encode writes 72 MiB per set
    assert bench.buffer_sets(wc, 1152 * wc.n // 2048, 512) == 8
    w3 = W.WORKLOADS["int3_r8_bf16_1024x8192"]             # reduce writes 3.5 + 16 MiB per set
    assert bench.buffer_sets(w3, 896 * w3.n // 2048, 512) == 27
    w2 = W.WORKLOADS["int3_bf16_codec_8m"]                 # decode reads 3.5 MiB per set
    assert bench.buffer_sets(w2, 896 * w2.n // 2048, 512) == 147
    w6 = W.WORKLOADS["int6_r8_fp16_32x1024x4096"]          # INT8 re-encoded sum: 136 + 256 MiB
    assert bench.buffer_sets(w6, 1152 * w6.n // 2048, 512, 2176 * w6.n // 2048) == 2
    tiny = W.small(wb, 2048)                               # capped
    assert bench.buffer_sets(tiny, 1152, 512) == bench.MAX_SETS
    for w, pb in ((wb, 1152 * wb.n // 2048), (wc, 1152 * wc.n // 2048), (w3, 896 * w3.n // 2048),
                  (w2, 896 * w2.n // 2048)):
        n = bench.buffer_sets(w, pb, 512)
        if w.reduce:
            reads = min(w.ranks * 2 * w.n, w.ranks * pb)
            writes = min(w.ranks * pb, pb + 2 * w.n)
        else:
            reads = writes = min(2 * w.n, pb)
        least = min(reads, writes)
        assert n * least >= 512 * mib > (n - 1) * least


def test_kernel_source_hash_covers_every_source_and_the_build_flags(monkeypatch):
    """Stored counter traffic is keyed to the build: any library source file,
    the compiler flags or a per-unit definition changes the key."""
    from bit_quantized_all_amd import build as hip_build
    srcs = bench.kernel_sources()
    csrc = os.path.join(ROOT, "bit_quantized_all_amd", "csrc")
    assert set(os.path.join("bit_quantized_all_amd", "csrc", f) for f in os.listdir(csrc)) <= set(srcs)
    assert "include/qr.h" in srcs
    base = bench.kernel_source_hash()
    monkeypatch.setattr(hip_build, "FLAGS", hip_build.FLAGS + ["-DQR_RED_GROUPS_PER_CU_MAX=3"])
    assert bench.kernel_source_hash() != base
    monkeypatch.undo()
    assert bench.kernel_source_hash() == base
    monkeypatch.setattr(hip_build, "SOURCES", hip_build.SOURCES[:-1])
    assert bench.kernel_source_hash() != base


def test_kernel_source_hash_is_the_same_for_a_copy_of_the_tree(monkeypatch):
    """The build's flags name include directories by absolute path; the key
    takes them relative to the repository, so a copy of the tree at another
    path (where the benchmark runs) finds the counters stored here."""
    from bit_quantized_all_amd import build as hip_build
    base = bench.kernel_source_hash()
    other = "/elsewhere/copy"

    def moved(a):
        return other + a[len(hip_build.ROOT):] if isinstance(a, str) and a.startswith(hip_build.ROOT) else a
    monkeypatch.setattr(hip_build, "FLAGS", [moved(f) for f in hip_build.FLAGS])
    monkeypatch.setattr(hip_build, "SOURCES", [(moved(s), d) for s, d in hip_build.SOURCES])
    monkeypatch.setattr(hip_build, "ROOT", other)
    assert any(f.startswith(other) for f in hip_build.FLAGS)
    assert bench.kernel_source_hash() == base
