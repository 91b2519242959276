#!/usr/bin/env python3
"""Throughput of encode -> compressed-domain reduce -> decode on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: R encodes (one per simulated rank, qr_encode) and one
fused qr_reduce_compressed that decodes the R packed buffers, sums them in
fp32 in rank order, re-encodes the sum and decodes it.  For the encode/decode
only workload a step is one qr_encode and one qr_decode.

The reported value is GB/s of FP16 input: R * n * 2 bytes per step divided by
the step time.  Alongside: the pipeline's algorithmic HBM bytes as % of the
MI355X peak (8 TB/s), the dominant kernel's roofline (average launch duration
from HIP events on the launch stream), and the CPU oracle timed on a bounded
sample of the same input.  With --graph the timed launches are captured in
HIP graphs and replayed, which removes the host-side cost of issuing each
launch from Python (it bounds steps on small messages).

Untimed warmup: at least W whole steps, and whole steps until at least
--min-warmup-ms (default 200) have passed; the line reports both W and the
number of warmup steps run.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of FP16 input through encode+compressed-reduce+decode; % HBM peak"
PEAK_HBM_GBS = 8000.0
TILE_BYTES = {"int3": 896, "int4": 1152, "int8": 2176, "asym4": 1072, "asym8": 2096, "fp4": 1152}
FORMAT_IDS = {"int3": 3, "int4": 4, "int8": 8, "asym4": 20, "asym8": 24, "fp4": 36}
KERNEL_SOURCE_DIR = "bit_quantized_all_amd/csrc"


def kernel_sources():
    """Every source file the library is built from (relative paths, sorted),
    with the C ABI header."""
    d = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    return sorted(os.path.join(KERNEL_SOURCE_DIR, f) for f in os.listdir(d)) + ["include/qr.h"]


def kernel_source_hash():
    """Hash of the library as built: every source file and the compiler flags
    and per-unit definitions of bit_quantized_all_amd/build.py.  Stored counter
    results apply only to a build with the same hash."""
    from bit_quantized_all_amd import build as hip_build

    h = hashlib.sha256()
    for p in kernel_sources():
        h.update(p.encode())
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    # paths inside the repository enter relative to it, so a copy of the tree
    # elsewhere has the same hash
    def rel(a):
        return os.path.relpath(a, hip_build.ROOT) if os.path.isabs(a) else a
    h.update(repr([rel(f) for f in hip_build.FLAGS]).encode())
    h.update(repr([(rel(src), defs) for src, defs in hip_build.SOURCES]).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes each kernel must move per launch (compressed buffers in HBM are the wire)."""
    c = TILE_BYTES[w.fmt] / 2048
    co = TILE_BYTES[w.out_fmt] / 2048
    n = w.n
    out = {"encode": n * (2 + c), "decode": n * (c + 2)}
    out["reduce"] = n * (w.ranks * c + co + 2)
    return out


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def traffic_from_profiles(kernel, workload):
    """Measured HBM bytes per launch from the committed counter summary, or None
    when there is none for this workload or it was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        d = json.load(f).get(workload)
    if not d or d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch", {}).get(kernel)


MAX_SETS = 1024


def set_traffic(w, pb, pbo=None):
    """Smallest per-kernel read and write footprint of one buffer set: the
    encodes read the R inputs of a set and write its R packed buffers, the
    reduce reads the R packed buffers and writes the re-encoded sum and y,
    the decode reads one packed buffer and writes y."""
    pbo = pb if pbo is None else pbo
    if w.reduce:
        reads = min(w.ranks * 2 * w.n, w.ranks * pb)
        writes = min(w.ranks * pb, pbo + 2 * w.n)
    else:
        reads = min(2 * w.n, pb)
        writes = min(pb, 2 * w.n)
    return reads, writes


def buffer_sets(w, pb, rotate_mib, pbo=None):
    """Number of identical buffer sets to rotate through: enough that each
    kernel's reads, and its writes, over one pass of the sets add up to
    rotate_mib MiB, at most MAX_SETS.  A launch's inputs were then last read,
    and its outputs last written, that many bytes of the kernel's own traffic
    ago, beyond what the 256 MB last-level cache holds: no launch reads its
    inputs from the cache, and no output still dirty in the cache is written
    again (which would spare its HBM write)."""
    reads, writes = set_traffic(w, pb, pbo)
    return max(1, min(MAX_SETS, -(-(rotate_mib << 20) // min(reads, writes))))


KERNEL_KEYS = {"encode": "encode_kernel", "reduce": "reduce_kernel", "decode": "decode_kernel"}
COPY_KEY = "copy_kernel"   # torch's device copy kernel (the calibration copy of --copy-ref)


def ingest_pmc(fetch_csv, write_csv, workload):
    """HBM bytes per launch of each kernel from two rocprofv3 counter runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --copy-ref --workload W`, each scaled so that the calibration copy
    (n * 2 bytes read, n * 2 written) reads as its known size.  Stored under
    the workload's name in profiles/hbm_traffic.json with the hash of the
    kernel sources."""
    import csv
    import statistics

    import workloads as W

    w = W.WORKLOADS[workload]

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                # this library's kernels only (torch has a reduce_kernel of its own)
                key = next((k for k, v in KERNEL_KEYS.items() if "qr::" + v in name), None)
                if key is None and "copy" in name.lower():
                    key = "copy"
                if key:
                    vals.setdefault(key, []).append(float(row["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    known = w.n * 2
    f_scale = known / (fetch["copy"] * 1024)
    w_scale = known / (write["copy"] * 1024)
    out = {"kernel_source_hash": kernel_source_hash(),
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
           "bytes_per_launch": {k: round(fetch[k] * 1024 * f_scale + write[k] * 1024 * w_scale)
                                for k in fetch if k in write and k != "copy"},
           "algorithmic_bytes_per_launch": {k: int(v) for k, v in algorithmic_bytes(w).items()}}
    allw = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            allw = json.load(f)
        if "kernel_source_hash" in allw:   # single-workload layout of older summaries
            allw = {}
    allw[workload] = out
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(allw, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


def _oracle_pass(o, w, host, a, b):
    """Oracle encode of tiles [a, b) of every rank, then its reduce (or decode)."""
    sv = slice(a * 2048, b * 2048)
    packed = [o.encode(FORMAT_IDS[w.fmt], w.io_dtype, h[sv]) for h in host]
    if w.reduce:
        return o.reduce_mixed(FORMAT_IDS[w.fmt], FORMAT_IDS[w.out_fmt], w.io_dtype, packed, (b - a) * 2048)
    return None, o.decode(FORMAT_IDS[w.fmt], w.io_dtype, packed[0], (b - a) * 2048)


def cpu_threads():
    """Host threads for the threaded oracle leg: the usable CPUs, at most 16."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return max(1, min(16, usable))


def cpu_baseline(w, xs, out, y, seconds, threads):
    """The oracle (plain C through ctypes, which releases the GIL) on the first
    tiles of every rank buffer, sized so that one single-threaded pass takes
    about seconds / 5.  Two legs, each the median of 5 passes: one thread, then
    the same tiles split into contiguous ranges over `threads` threads.  The
    inputs are copied to the host before any timing.  The single-threaded
    outputs are compared with the GPU's bytes for the same tiles, and the
    threaded outputs with the single-threaded ones."""
    import statistics
    import threading

    import numpy as np
    import torch

    import oracle

    o = oracle.default()
    tb = TILE_BYTES[w.out_fmt]
    ntiles = w.n // 2048
    probe = min(16, ntiles)
    host = [x[:probe * 2048].view(torch.int16).cpu().numpy().view(np.uint16) for x in xs]
    t0 = time.perf_counter()
    _oracle_pass(o, w, host, 0, probe)
    per_tile = (time.perf_counter() - t0) / probe
    tiles = max(probe, min(ntiles, int(seconds / 5 / per_tile) // 16 * 16))
    host = [x[:tiles * 2048].view(torch.int16).cpu().numpy().view(np.uint16) for x in xs]

    single = []
    for _ in range(5):
        t0 = time.perf_counter()
        po, yo = _oracle_pass(o, w, host, 0, tiles)
        single.append(time.perf_counter() - t0)
    ok = bool(np.array_equal(yo, y[:tiles * 2048].view(torch.int16).cpu().numpy().view(np.uint16)))
    if po is not None:
        ok &= bool(np.array_equal(po, out[:tiles * tb].cpu().numpy()))

    threads = max(1, min(threads, tiles))
    bounds = [tiles * k // threads for k in range(threads + 1)]
    multi = []
    for _ in range(5):
        parts = [None] * threads

        def work(k):
            parts[k] = _oracle_pass(o, w, host, bounds[k], bounds[k + 1])

        pool = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
        t0 = time.perf_counter()
        for t in pool:
            t.start()
        for t in pool:
            t.join()
        multi.append(time.perf_counter() - t0)
    ok &= bool(np.array_equal(np.concatenate([p[1] for p in parts]), yo))
    if po is not None:
        ok &= bool(np.array_equal(np.concatenate([p[0] for p in parts]), po))

    fp16_bytes = w.ranks * tiles * 2048 * 2
    t1, tn = statistics.median(single), statistics.median(multi)
    what = (f"first {tiles} tiles ({tiles * 2048} values) of each of the {w.ranks} rank buffers of "
            f"{w.name}: oracle encode x{w.ranks} + " + ("reduce with decode" if w.reduce else "decode")
            + f"; median of 5 passes; one pass takes {t1:.2f} s on one thread")
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(fp16_bytes / tn / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": what + f", {tn:.3f} s on {threads} threads over contiguous tile ranges",
            "single_thread": {"value": round(fp16_bytes / t1 / 1e9, 5), "unit": "GB/s", "cores": 1},
            "cpu_model": model, "host_cpus": os.cpu_count()}, ok


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warmup-ms", type=float, default=200.0,
                    help="after the W warmup steps, keep running untimed whole steps until this much "
                         "time has passed since the warmup began: the first tens of milliseconds of "
                         "full-size steps run up to 3%% slower while the GPU settles")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--values", type=int, default=None,
                    help="override the workload's values per rank (a multiple of 2048), e.g. for a "
                         "message-size sweep; the distribution and the rank count stay")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="single-threaded oracle time of the 5 timed passes together (the threaded "
                         "leg adds as much CPU time again)")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="threads of the threaded oracle leg (default: usable CPUs, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-mib", type=int, default=512,
                    help="rotate through enough identical buffer sets (inputs, packed, outputs) that "
                         "every kernel reads, and writes, at least this many MiB over one pass of "
                         "the sets, so that the 256 MB last-level cache can neither serve a launch's "
                         "reads nor absorb its writes from an earlier launch "
                         f"(at most {MAX_SETS} sets)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed launches in HIP graphs and replay them (removes the "
                         "host-side launch cost that bounds small messages)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also time a plain device copy of one rank's input (bandwidth reference and "
                         "calibration kernel for the HBM traffic counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--lib", default=None,
                    help="load the libqr.so at PATH instead of the package's (a compile-time variant "
                         "made with python -m bit_quantized_all_amd.build --out PATH -DNAME=VALUE)")
    args = ap.parse_args()

    if args.ingest_pmc:
        import workloads as W
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload or W.BENCH_WORKLOAD)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the sharded "
              "two-shot exchange is described, not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_all_amd as qa
    import workloads as W

    if args.lib:
        from bit_quantized_all_amd import qr as _qr
        _qr.LIB_PATH = os.path.abspath(args.lib)
    name = args.workload or W.BENCH_WORKLOAD
    w = W.WORKLOADS[name]
    if args.values is not None:
        if args.values <= 0 or args.values % 2048:
            print("--values must be a positive multiple of 2048", file=sys.stderr)
            sys.exit(2)
        w = W.small(w, args.values)
    qa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    pb = qa.qr_packed_bytes(w.fmt, w.n)
    pbo = qa.qr_packed_bytes(w.out_fmt, w.n)
    set_bytes = w.ranks * (2 * w.n + pb) + (pbo if w.reduce else 0) + 2 * w.n
    nsets = buffer_sets(w, pb, args.rotate_mib, pbo)

    class BufferSet:
        def __init__(self, xs):
            self.xs = xs
            self.packed = [torch.empty(pb, dtype=torch.uint8, device=dev) for _ in range(w.ranks)]
            self.out = torch.empty(pbo, dtype=torch.uint8, device=dev) if w.reduce else None
            self.y = torch.empty(w.n, dtype=w.dtype, device=dev)

    xs = W.inputs(w, seed=args.seed, device=dev)
    sets = [BufferSet(xs)] + [BufferSet([x.clone() for x in xs]) for _ in range(nsets - 1)]
    torch.cuda.synchronize()

    # Every launch goes to the current stream: the timing stream when eager, the
    # capture stream while a graph is being recorded.
    def encode(b, r):
        qa.qr_encode(w.fmt, b.xs[r], b.packed[r])

    def finish(b):
        if w.reduce:
            qa.qr_reduce_compressed_mixed(w.fmt, w.out_fmt, w.dtype, b.packed, w.n, packed_out=b.out, y_out=b.y)
        else:
            qa.qr_decode(w.fmt, b.packed[0], w.n, w.dtype, y=b.y)

    def step(b):
        for r in range(w.ranks):
            encode(b, r)
        finish(b)

    def runner(fn):
        """fn itself (eager), or a function that replays fn captured in a HIP graph."""
        if not args.graph:
            return fn
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g.replay

    t_warm = time.perf_counter()
    warm_steps = max(args.warmup, nsets)
    for i in range(warm_steps):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    while (time.perf_counter() - t_warm) * 1e3 < args.min_warmup_ms:
        for _ in range(nsets):
            step(sets[warm_steps % nsets])
            warm_steps += 1
        torch.cuda.synchronize()
    run_steps = [runner(lambda b=b: step(b)) for b in sets]
    for run in run_steps:
        run()
    torch.cuda.synchronize()

    # host-side markers (roctx under ROCm) around the timed regions, for traces
    # taken with rocprofv3 --marker-trace; a no-op where torch has none
    import contextlib

    def marker(label):
        rng = getattr(getattr(torch.cuda, "nvtx", None), "range", None)
        return rng(label) if rng is not None else contextlib.nullcontext()

    # timed region 1: K clean steps between two events, rotating the buffer sets
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with marker(f"qr.steps x{args.steps}"):
        start.record(stream)
        for i in range(args.steps):
            run_steps[i % nsets]()
        end.record(stream)
        torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # the same K steps again, with an event between consecutive steps -> median step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with marker(f"qr.steps_with_events x{args.steps}"):
        evs[0].record(stream)
        for i in range(args.steps):
            run_steps[i % nsets]()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[args.steps // 2] if args.steps % 2 else \
        0.5 * (per_step[args.steps // 2 - 1] + per_step[args.steps // 2])

    # timed region 2: each kernel alone, K steps' worth of back-to-back launches
    # between two events on the launch stream -> average launch duration
    def timed(label, fn, launches):
        run = runner(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with marker(f"qr.{label} x{launches}"):
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches * 1e3

    kname = "reduce" if w.reduce else "decode"
    kern_us = {
        "encode": timed("encode", lambda: [encode(sets[i % nsets], r) for i in range(args.steps)
                                           for r in range(w.ranks)], args.steps * w.ranks),
        kname: timed(kname, lambda: [finish(sets[i % nsets]) for i in range(args.steps)], args.steps),
    }
    run_steps[0]()   # the outputs checked below come from one whole step on set 0
    torch.cuda.synchronize()
    packed, out, y = sets[0].packed, sets[0].out, sets[0].y
    print(f"# {name}: {ms_per_step:.4f} ms/step; per-launch us: "
          + ", ".join(f"{k}={v:.2f}" for k, v in kern_us.items()), file=sys.stderr, flush=True)

    copy_ref = None
    if args.copy_ref:
        src, dst = xs[0], torch.empty_like(xs[0])
        dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        us = c0.elapsed_time(c1) / args.steps * 1e3
        copy_ref = {"bytes": 4 * w.n, "us_per_launch": round(us, 3), "gbs": round(4 * w.n / us / 1e3, 1)}
        del dst

    # quality: RMSE of the decoded result against the unquantized fp32 sum of
    # the inputs (rank order), absolute and relative to the RMS of that sum
    ref = xs[0].float()
    for r in range(1, w.ranks):
        ref += xs[r].float()
    if not w.reduce:
        ref = xs[0].float()
    err = (y.float() - ref).pow(2).mean().sqrt().item()
    rms = ref.pow(2).mean().sqrt().item()
    rmse = {"abs": err, "rel": err / rms if rms else None}
    del ref

    ab = algorithmic_bytes(w)
    launches = {"encode": w.ranks, "reduce": 1 if w.reduce else 0, "decode": 0 if w.reduce else 1}
    step_bytes = sum(ab[k] * launches[k] for k in launches)
    fp16_input = w.ranks * w.n * 2
    value = fp16_input / (ms_per_step * 1e-3) / 1e9
    pipe_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    # stored counter traffic belongs to the default build of the current sources
    traffic = (lambda k: None) if args.lib else (lambda k: traffic_from_profiles(k, name))
    kernels = {}
    for k, us in kern_us.items():
        g = ab[k] / (us * 1e-6) / 1e9
        kernels[k] = {"us_per_launch": round(us, 3), "launches_per_step": launches[k],
                      "algorithmic_bytes": int(ab[k]), "achieved_gbs": round(g, 1),
                      "frac": round(g / PEAK_HBM_GBS, 4), "traffic": traffic(k)}
    dom = max(kern_us, key=lambda k: kern_us[k] * launches[k])
    roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["achieved_gbs"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kernels[dom]["frac"],
                "traffic": traffic(dom)}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "launch": "hip_graph" if args.graph else "eager",
        "config": {"workload": name, "format": w.fmt, "format_out": w.out_fmt, "io_dtype": w.io_dtype,
                   "ranks": w.ranks,
                   "values_per_rank": w.n, "shape": list(w.shape), "seed": args.seed,
                   "buffer_sets": nsets, "set_mib": round(set_bytes / 2 ** 20, 1)},
        "pct_hbm_peak": round(100 * pipe_gbs / PEAK_HBM_GBS, 2),
        "pipeline_hbm_gbs": round(pipe_gbs, 1),
        "roofline": roofline,
        "kernels": kernels,
        "rmse_vs_fp32_sum": rmse,
    }
    if copy_ref:
        result["copy_ref"] = copy_ref
    if args.lib:
        result["library"] = os.path.abspath(args.lib)
    ok = True
    if not args.no_cpu_baseline:
        cb, ok = cpu_baseline(w, xs, out, y, args.cpu_seconds, args.cpu_threads or cpu_threads())
        result["cpu_baseline"] = cb
        result["parity_sample"] = ok
    print(json.dumps(result), flush=True)
    if not ok:
        print("bench.py: the GPU output differs from the oracle on the sampled tiles", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
