"""Parity of the HIP path with the CPU oracle (MI355X only).

Every comparison is element by element on the same seeded inputs: packed
codes and scales must be bit-identical, and decoded / reduced fp16/bf16
outputs bit-identical as well (the acceptance bar allows 1 ulp of the output
dtype for those; every step is a correctly rounded IEEE operation, so exact
equality is what is expected and what is asserted).  Sizes span several
tiles, waves and workgroups, with a ragged last workgroup; the full-size
workloads are checked on sampled tiles, which the oracle computes one by one
(tiles are independent), plus properties that hold at any size, and the bench
workload and the INT3 two-rank reduce on every tile of seed 0.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle_pins as P
import workloads as W

pytestmark = pytest.mark.gpu

FMTS = ("int3", "int4", "int8")
AFMTS = ("asym4", "asym8")
BITS = {"int3": 3, "int4": 4, "int8": 8, "asym4": 20, "asym8": 24, "fp4": 36}   # oracle format ids
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_all_amd as qa
    qa.lib()
    assert torch.cuda.is_available()
    return qa


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a, dtype=None):
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(dtype)
    else:
        t = torch.from_numpy(a.copy())
    return t.cuda()


def gen(kind, dtype, n, seed):
    """Host fp16/bf16 bit patterns for a named value family."""
    rng = np.random.default_rng(seed)
    nb = n // 32
    if kind == "normal":
        x = rng.standard_normal(n)
    elif kind == "outliers":
        x = rng.standard_normal(n)
        x[rng.random(n) < 0.001] *= 50
    elif kind == "scales":      # block scales spread over many binades, incl. fp16 subnormal scales
        x = rng.standard_normal((nb, 32)) * np.exp(rng.uniform(-14, 9, size=(nb, 1)))
    elif kind == "specials":    # zero blocks, -0, tiny, huge and exact multiples of a scale
        x = rng.standard_normal((nb, 32))
        sel = rng.integers(0, 6, nb)
        x[sel == 0] = 0.0
        x[sel == 1] = -0.0
        x[sel == 2] *= 2.0 ** -20
        x[sel == 3] = rng.integers(-8, 8, size=(int((sel == 3).sum()), 32)) * 0.25
        x[sel == 4] *= 3000.0
        x = x.ravel()
    else:
        raise ValueError(kind)
    x = np.asarray(x, np.float64).ravel()
    if dtype == "fp16":
        return P.f16_bits(np.clip(x, -65504, 65504))
    return P.bf16_bits(x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# encode / decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ntiles", [1, 5, 37, 1031])
@pytest.mark.parametrize("kind", ["normal", "outliers", "scales", "specials"])
def test_encode_decode_parity(qa, oracle, fmt, dtype, ntiles, kind):
    n = ntiles * 2048
    xb = gen(kind, dtype, n, seed=ntiles * 7 + len(kind))
    log(f"encode/decode {fmt} {dtype} tiles={ntiles} {kind}")
    x = dev(xb, DT[dtype])
    p = qa.qr_encode(fmt, x)
    y = qa.qr_decode(fmt, p, n, DT[dtype])
    torch.cuda.synchronize()
    want_p = oracle.encode(BITS[fmt], dtype, xb)
    got_p = p.cpu().numpy()
    if not np.array_equal(got_p, want_p):
        gc, gs = P.unpack(BITS[fmt], got_p)
        wc, ws = P.unpack(BITS[fmt], want_p)
        bad = np.argwhere(gc != wc)
        raise AssertionError(f"codes differ at {bad[:5].tolist()} (scales equal: {np.array_equal(gs, ws)})")
    want_y = oracle.decode(BITS[fmt], dtype, want_p, n)
    assert np.array_equal(u16(y), want_y)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_decode_arbitrary_packed(qa, oracle, fmt, dtype):
    """Decode of packed data that no encoder produced: every code, every
    finite fp16 scale (normal, subnormal, zero)."""
    bits = BITS[fmt]
    rng = np.random.default_rng(bits)
    T = 517
    codes = rng.integers(0, 1 << bits, size=(T, 2048))
    sb = rng.integers(0, 0x7C00, size=(T, 64)).astype(np.uint16)
    sb[:, :3] = [0, 1, 0x7BFF]
    packed = P.pack(bits, codes, sb)
    log(f"decode arbitrary {fmt} {dtype}")
    y = qa.qr_decode(fmt, dev(packed), T * 2048, DT[dtype])
    torch.cuda.synchronize()
    assert np.array_equal(u16(y), oracle.decode(bits, dtype, packed, T * 2048))


# ---------------------------------------------------------------------------
# fused reduction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 11, 15, 16])
@pytest.mark.parametrize("ntiles", [3, 133])
def test_reduce_parity(qa, oracle, fmt, dtype, R, ntiles):
    bits = BITS[fmt]
    n = ntiles * 2048
    kinds = ["normal", "outliers", "scales", "specials"]
    xs = [gen(kinds[r % 4], dtype, n, seed=1000 * R + 10 * r + ntiles) for r in range(R)]
    log(f"reduce {fmt} {dtype} R={R} tiles={ntiles}")
    packed = [qa.qr_encode(fmt, dev(x, DT[dtype])) for x in xs]
    out, y = qa.qr_reduce_compressed(fmt, DT[dtype], packed, n)
    out2, none = qa.qr_reduce_compressed(fmt, DT[dtype], packed, n, with_output=False)
    torch.cuda.synchronize()
    assert none is None
    wranks = [oracle.encode(bits, dtype, x) for x in xs]
    for r in range(R):
        assert np.array_equal(packed[r].cpu().numpy(), wranks[r]), r
    wout, wy = oracle.reduce(bits, dtype, wranks, n)
    got = out.cpu().numpy()
    if not np.array_equal(got, wout):
        gc, gs = P.unpack(bits, got)
        wc, ws = P.unpack(bits, wout)
        raise AssertionError(f"re-encoded tile differs: codes at {np.argwhere(gc != wc)[:5].tolist()}, "
                             f"scales at {np.argwhere(gs != ws)[:5].tolist()}")
    assert np.array_equal(u16(y), wy)
    assert np.array_equal(out2.cpu().numpy(), wout)


def test_reduce_repeated_rank_buffer(qa, oracle):
    """The same buffer passed for several ranks (inputs may alias each other)."""
    n = 9 * 2048
    xb = gen("normal", "fp16", n, 3)
    p = qa.qr_encode("int4", dev(xb, torch.float16))
    out, y = qa.qr_reduce_compressed("int4", torch.float16, [p, p, p], n)
    torch.cuda.synchronize()
    wp = oracle.encode(4, "fp16", xb)
    wout, wy = oracle.reduce(4, "fp16", [wp, wp, wp], n)
    assert np.array_equal(out.cpu().numpy(), wout) and np.array_equal(u16(y), wy)


def test_reduce_fp16_overflow(qa, oracle):
    """An fp16 sum above 65504 rounds to inf; the re-encode saturates the scale
    at 65504 and the codes at the ends of the range, on both sides."""
    n = 2 * 2048
    xb = [P.f16_bits(np.full(n, 60000.0 * (1 if r % 2 == 0 else 1))) for r in range(4)]
    xb[1][::3] = P.f16_bits(-60000.0)
    log("reduce fp16 overflow")
    packed = [qa.qr_encode("int4", dev(x, torch.float16)) for x in xb]
    out, y = qa.qr_reduce_compressed("int4", torch.float16, packed, n)
    torch.cuda.synchronize()
    wout, wy = oracle.reduce(4, "fp16", [oracle.encode(4, "fp16", x) for x in xb], n)
    assert np.array_equal(out.cpu().numpy(), wout) and np.array_equal(u16(y), wy)


def test_golden_rank_order_on_gpu(qa):
    """The hand-derived rank-order example (tests/golden/reduce_rank_order.txt)."""
    scale, elems = P._golden_expect("reduce_rank_order.txt")
    vals = np.zeros((4, 2048))
    vals[0, [0, 2, 3]] = [-16, 2, 14]
    vals[1, [0, 1]] = [-2.0 ** -20, -2.0 ** -17]
    vals[2, [0, 2, 3]] = [14, -16, 2]
    vals[3, [0, 2, 3]] = [2, 14, -16]
    packed = [qa.qr_encode("int4", dev(P.f16_bits(v), torch.float16)) for v in vals]
    out, y = qa.qr_reduce_compressed("int4", torch.float16, packed, 2048)
    torch.cuda.synchronize()
    codes, sb = P.unpack(4, out.cpu().numpy())
    yb = u16(y)
    assert sb[0, 0] == scale
    for name, idx in (("A", 0), ("B", 1), ("E2", 2), ("E3", 3)):
        assert codes[0, idx] == elems[name][0] and yb[idx] == elems[name][1], name


# ---------------------------------------------------------------------------
# the workloads, at CPU-checkable size and at full size (sampled tiles)
# ---------------------------------------------------------------------------

def run_pipeline(qa, w, xs):
    packed = [qa.qr_encode(w.fmt, x) for x in xs]
    if not w.reduce:
        return packed, None, qa.qr_decode(w.fmt, packed[0], w.n, w.dtype)
    out, y = qa.qr_reduce_compressed_mixed(w.fmt, w.out_fmt, w.dtype, packed, w.n)
    return packed, out, y


def check_tiles(oracle, w, xs_host_tiles, packed, out, y, tiles):
    """Oracle on the given tiles of every rank vs the GPU's bytes there."""
    bits = BITS[w.fmt]
    tb = oracle.packed_bytes(bits, 2048)
    idx_b = np.concatenate([np.arange(t * tb, (t + 1) * tb) for t in tiles])
    idx_v = np.concatenate([np.arange(t * 2048, (t + 1) * 2048) for t in tiles])
    nt = len(tiles) * 2048
    wr = [oracle.encode(bits, w.io_dtype, xt) for xt in xs_host_tiles]
    for r in range(len(wr)):
        assert np.array_equal(packed[r][idx_b], wr[r]), f"rank {r} encode differs"
    if out is None:
        assert np.array_equal(y[idx_v], oracle.decode(bits, w.io_dtype, wr[0], nt))
        return
    obits = BITS[w.out_fmt]
    otb = oracle.packed_bytes(obits, 2048)
    idx_o = np.concatenate([np.arange(t * otb, (t + 1) * otb) for t in tiles])
    wout, wy = oracle.reduce_mixed(bits, obits, w.io_dtype, wr, nt)
    assert np.array_equal(out[idx_o], wout), "re-encoded sum differs"
    assert np.array_equal(y[idx_v], wy), "decoded sum differs"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_smallest_workload_exact(qa, oracle, seed):
    """The INT3 R=2 8192-value workload, every value, seeds 0..2."""
    w = W.WORKLOADS["int3_r2_fp16_8k"]
    xs = W.inputs(w, seed=seed)
    log(f"workload int3_r2_fp16_8k seed={seed}")
    packed, out, y = run_pipeline(qa, w, [x.cuda() for x in xs])
    torch.cuda.synchronize()
    check_tiles(oracle, w, [u16(x) for x in xs], [p.cpu().numpy() for p in packed],
                out.cpu().numpy(), u16(y), list(range(w.n // 2048)))


FULL_SIZE_CASES = [(k, seed) for k in W.WORKLOADS if k != "int3_r2_fp16_8k"
                   for seed in ((0,) if k.startswith("sweep_") else (0, 1, 2))]


@pytest.mark.parametrize("name,seed", FULL_SIZE_CASES)
def test_workload_full_size_sampled(qa, oracle, name, seed):
    w = W.WORKLOADS[name]
    log(f"workload {name} n={w.n} R={w.ranks} seed={seed}")
    xs = W.inputs(w, seed=seed, device="cuda")
    packed, out, y = run_pipeline(qa, w, xs)
    # a second run must give identical bytes (determinism)
    packed2, out2, y2 = run_pipeline(qa, w, xs)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(packed, packed2))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    if out is not None:
        assert torch.equal(out, out2)
        # the fused final decode equals the standalone decode of the re-encoded sum
        yd = qa.qr_decode(w.out_fmt, out, w.n, w.dtype)
        assert torch.equal(y.view(torch.int16), yd.view(torch.int16))
    ntiles = w.n // 2048
    rng = np.random.default_rng(ntiles + seed)
    tiles = sorted(set([0, 1, ntiles - 1, ntiles // 2] + list(rng.integers(0, ntiles, 60))))
    tb = oracle.packed_bytes(BITS[w.fmt], 2048)
    sel_v = torch.tensor(np.concatenate([np.arange(t * 2048, (t + 1) * 2048) for t in tiles]), device="cuda")
    sel_b = np.concatenate([np.arange(t * tb, (t + 1) * tb) for t in tiles])
    xs_t = [u16(x[sel_v]) for x in xs]
    packed_full = [p.cpu().numpy() for p in packed]
    y_host = np.zeros(w.n, np.uint16)
    y_host[sel_v.cpu().numpy()] = u16(y[sel_v])
    out_host = out.cpu().numpy() if out is not None else None
    del sel_b
    check_tiles(oracle, w, xs_t, packed_full, out_host, y_host, tiles)


# Workloads whose whole full-size output is checked against the oracle, tile
# by tile: the bench workload, the INT3 two-rank reduce, the mixed INT4 -> INT8
# and ASYM4 -> ASYM8 reduces, FP4, and INT8 at 512 MiB per rank (the kernels'
# large-grid launch choices: unordered decodes, residency caps).
EVERY_TILE_CASES = ["int4_r8_fp16_32x1024x4096", "int3_r2_fp16_32x1024x4096", "int6_r8_fp16_32x1024x4096",
                    "asym6_r8_fp16_32x1024x4096", "fp4_r8_fp16_32x1024x4096", "sweep_r4_fp16_int8_512mib"]


def _host_threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", EVERY_TILE_CASES)
def test_workload_full_size_every_tile(qa, oracle, name):
    """Every byte of the full-size outputs (each rank's packed buffer, the
    re-encoded sum and the decoded sum) of seed 0 against the oracle.  The
    oracle runs on the host over contiguous tile ranges in parallel threads
    (its C calls release the GIL)."""
    import threading

    w = W.WORKLOADS[name]
    log(f"every tile: workload {name} n={w.n} R={w.ranks} seed=0")
    xs = W.inputs(w, seed=0, device="cuda")
    packed, out, y = run_pipeline(qa, w, xs)
    torch.cuda.synchronize()
    xs_h = [u16(x) for x in xs]
    packed_h = [p.cpu().numpy() for p in packed]
    out_h, y_h = out.cpu().numpy(), u16(y)
    del xs, packed, out, y
    torch.cuda.empty_cache()
    bits, bits_out = BITS[w.fmt], BITS[w.out_fmt]
    tb, tbo = oracle.packed_bytes(bits, 2048), oracle.packed_bytes(bits_out, 2048)
    ntiles = w.n // 2048
    threads = _host_threads()
    bounds = [ntiles * k // threads for k in range(threads + 1)]
    bad = [None] * threads

    def work(k):
        a, b = bounds[k], bounds[k + 1]
        sv = slice(a * 2048, b * 2048)
        wr = [oracle.encode(bits, w.io_dtype, xh[sv]) for xh in xs_h]
        for r in range(w.ranks):
            if not np.array_equal(packed_h[r][a * tb:b * tb], wr[r]):
                bad[k] = f"rank {r} encode differs in tiles [{a}, {b})"
                return
        wout, wy = oracle.reduce_mixed(bits, bits_out, w.io_dtype, wr, (b - a) * 2048)
        if not np.array_equal(out_h[a * tbo:b * tbo], wout):
            bad[k] = f"re-encoded sum differs in tiles [{a}, {b})"
        elif not np.array_equal(y_h[sv], wy):
            bad[k] = f"decoded sum differs in tiles [{a}, {b})"

    pool = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    log(f"every tile: {ntiles} tiles checked on {threads} host threads")
    assert all(b is None for b in bad), [b for b in bad if b]


def test_block_scale_every_fp16_scale():
    """The library's block-scale device function over every positive finite
    fp16 scale d (block maximum Q*d): scale bits d and encode multiplier equal
    to the correctly rounded IEEE quotient 1.0f / d, for each format."""
    import ctypes
    import os
    lib = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_helpers", "libscale_check.so")
    L = ctypes.CDLL(lib)
    L.qr_test_scale_check.argtypes = [ctypes.c_void_p]
    counters = torch.zeros(6, dtype=torch.int32, device="cuda")
    log("scale check over all fp16 scales")
    assert L.qr_test_scale_check(counters.data_ptr()) == 0
    assert counters.cpu().tolist() == [0] * 6


def test_fp4_hardware_conversions_and_scale():
    """The FP4 device functions against definitions in the test helper: the
    gfx950 scaled FP4 conversion (scale 1.0) on every non-NaN fp32 pattern is
    the nearest E2M1 value with ties to an even mantissa, saturating at 6,
    sign kept, nibbles and byte position as the tile layout needs; the
    reverse conversion gives the E2M1 values for every byte and position; the
    FP4 block scale and multiplier are right for every fp16 and bf16 maximum."""
    import ctypes
    import os
    lib = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_helpers", "libscale_check.so")
    L = ctypes.CDLL(lib)
    L.qr_test_fp4_check.argtypes = [ctypes.c_void_p]
    counters = torch.tensor([0, -1, 0, 0, 0], dtype=torch.int32, device="cuda")
    log("fp4 conversions: every fp32 pattern, every byte, every fp16/bf16 block maximum")
    assert L.qr_test_fp4_check(counters.data_ptr()) == 0
    c = counters.cpu().tolist()
    assert c == [0, -1, 0, 0, 0], f"mismatches {c[0]} (first pattern {c[1] & 0xFFFFFFFF:#010x}), unpack {c[2]}, scale fp16 {c[3]} bf16 {c[4]}"


MIXED = [("int4", "int8"), ("int3", "int4"), ("int3", "int8"), ("int4", "int3"), ("int8", "int3"),
         ("int8", "int4")]


@pytest.mark.parametrize("fi,fo", MIXED)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 5, 8, 16])
def test_reduce_mixed_parity(qa, oracle, fi, fo, dtype, R):
    """Inputs in one format, the re-encoded sum in another ("INT6" = INT4 -> INT8)."""
    n = 37 * 2048
    kinds = ["normal", "outliers", "scales", "specials"]
    xs = [gen(kinds[r % 4], dtype, n, seed=77 * R + r) for r in range(R)]
    log(f"reduce mixed {fi}->{fo} {dtype} R={R}")
    packed = [qa.qr_encode(fi, dev(x, DT[dtype])) for x in xs]
    out, y = qa.qr_reduce_compressed_mixed(fi, fo, DT[dtype], packed, n)
    out2, _ = qa.qr_reduce_compressed_mixed(fi, fo, DT[dtype], packed, n, with_output=False)
    torch.cuda.synchronize()
    assert out.numel() == P.tile_bytes(BITS[fo]) * (n // 2048)
    wout, wy = oracle.reduce_mixed(BITS[fi], BITS[fo], dtype, [oracle.encode(BITS[fi], dtype, x) for x in xs], n)
    assert np.array_equal(out.cpu().numpy(), wout)
    assert np.array_equal(u16(y), wy)
    assert np.array_equal(out2.cpu().numpy(), wout)


@pytest.mark.parametrize("fi,fo", [("int4", "int4"), ("int8", "int8"), ("int4", "int8")])
@pytest.mark.parametrize("ntiles", [16384, 16385])
def test_reduce_both_sides_of_the_decode_order_switch(qa, oracle, fi, fo, ntiles):
    """INT4 and INT8 inputs reduce with rank-ordered decodes up to 16384 tiles
    and unordered ones above (a launch-time choice between two kernels): both
    sides, every byte against the oracle."""
    n = ntiles * 2048
    R = 3
    kinds = ["normal", "outliers", "scales"]
    xs = [gen(kinds[r], "fp16", n, seed=5 * ntiles + r) for r in range(R)]
    log(f"reduce {fi}->{fo} fp16 R={R} tiles={ntiles}")
    packed = [qa.qr_encode(fi, dev(x, torch.float16)) for x in xs]
    out, y = qa.qr_reduce_compressed_mixed(fi, fo, torch.float16, packed, n)
    torch.cuda.synchronize()
    wranks = [oracle.encode(BITS[fi], "fp16", x) for x in xs]
    wout, wy = oracle.reduce_mixed(BITS[fi], BITS[fo], "fp16", wranks, n)
    assert np.array_equal(out.cpu().numpy(), wout)
    assert np.array_equal(u16(y), wy)


def test_empty_calls_are_size_errors(qa):
    """n = 0 through every entry point: rejected with QR_ERR_SIZE on the host
    (the tile is the unit), nothing is launched."""
    e16 = torch.empty(0, dtype=torch.float16, device="cuda")
    e8 = torch.empty(0, dtype=torch.uint8, device="cuda")
    calls = [lambda: qa.qr_encode("int4", e16, e8),
             lambda: qa.qr_decode("int3", e8, 0, torch.float16, y=e16),
             lambda: qa.qr_reduce_compressed("int8", torch.bfloat16, [e8, e8], 0, packed_out=e8,
                                             y_out=torch.empty(0, dtype=torch.bfloat16, device="cuda")),
             lambda: qa.qr_reduce_compressed_mixed("int4", "int8", torch.float16, [e8], 0, packed_out=e8,
                                                   y_out=e16)]
    for call in calls:
        with pytest.raises(qa.QRError) as ei:
            call()
        assert ei.value.status == qa.QR_ERR_SIZE
    torch.cuda.synchronize()


def test_misaligned_and_aliased_device_buffers(qa):
    """Real device buffers with an offset of 2 bytes, and an output inside an
    input: rejected on the host, nothing is launched."""
    x = torch.zeros(2048 * 2 + 8, dtype=torch.float16, device="cuda")
    p = torch.empty(1152 * 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(qa.QRError) as ei:
        qa.qr_encode("int4", x[1:2049], p[:1152])
    assert ei.value.status == 3
    with pytest.raises(qa.QRError) as ei:
        qa.qr_reduce_compressed("int4", torch.float16, [p[:1152]], 2048, packed_out=p[:1152], y_out=x[:2048])
    assert ei.value.status == 5
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# asymmetric group codec (128-value groups, scale + zero point)
# ---------------------------------------------------------------------------

def gen_groups(dtype, n, seed):
    """Host fp16/bf16 bit patterns with one structure per 128-value group:
    zero, one-signed (all positive / all negative), a range held by a single
    32-value block (the group range crosses lanes), fp16-subnormal ranges
    (zero-point clamp), huge magnitudes (scale saturation for bf16), a
    shifted mean, and exact grid points (q - z) * 2^m."""
    rng = np.random.default_rng(seed)
    ng = n // 128
    x = rng.standard_normal((ng, 128))
    sel = rng.integers(0, 9, ng)
    x[sel == 0] = 0.0
    x[sel == 1] = np.abs(x[sel == 1]) * 3
    x[sel == 2] = -np.abs(x[sel == 2]) * 0.3
    k = int((sel == 3).sum())
    if k:
        x[sel == 3] *= 1e-3
        lane = rng.integers(0, 4, k)
        rows = np.nonzero(sel == 3)[0]
        for r, l in zip(rows, lane):
            x[r, 32 * l:32 * l + 32] *= 4000.0
    k = int((sel == 4).sum())
    if k:
        x[sel == 4] = rng.integers(-400, 60, size=(k, 128)) * 2.0 ** -24
    x[sel == 5] *= 2.0 ** 30 if dtype == "bf16" else 20000.0
    x[sel == 6] = x[sel == 6] + 3.0
    k = int((sel == 7).sum())
    if k:
        x[sel == 7] = (rng.integers(0, 16, size=(k, 128)) - 5) * 2.0 ** rng.integers(-8, 3, size=(k, 1))
    x[sel == 8] = -0.0
    x = x.ravel()
    if dtype == "fp16":
        return P.f16_bits(np.clip(x, -65504, 65504))
    return P.bf16_bits(x.astype(np.float32).astype(np.float64))


def agen(kind, dtype, n, seed):
    return gen_groups(dtype, n, seed) if kind == "groups" else gen(kind, dtype, n, seed)


def first_diff(got, want):
    bad = np.nonzero(got != want)[0]
    return bad[:8].tolist()


@pytest.mark.parametrize("fmt", AFMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ntiles", [1, 5, 37, 1031])
@pytest.mark.parametrize("kind", ["normal", "outliers", "scales", "groups"])
def test_asym_encode_decode_parity(qa, oracle, fmt, dtype, ntiles, kind):
    n = ntiles * 2048
    xb = agen(kind, dtype, n, seed=ntiles * 13 + len(kind))
    log(f"asym encode/decode {fmt} {dtype} tiles={ntiles} {kind}")
    p = qa.qr_encode(fmt, dev(xb, DT[dtype]))
    y = qa.qr_decode(fmt, p, n, DT[dtype])
    torch.cuda.synchronize()
    want_p = oracle.encode(BITS[fmt], dtype, xb)
    got_p = p.cpu().numpy()
    assert got_p.size == want_p.size
    assert np.array_equal(got_p, want_p), f"packed bytes differ at {first_diff(got_p, want_p)}"
    assert np.array_equal(u16(y), oracle.decode(BITS[fmt], dtype, want_p, n))


@pytest.mark.parametrize("fmt", AFMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_asym_decode_arbitrary_packed(qa, oracle, fmt, dtype):
    """Decode of packed data no encoder produced: every code, zero points over
    [0, 2^b - 1], every finite fp16 scale class (zero, subnormal, largest)."""
    bits = 4 if fmt == "asym4" else 8
    rng = np.random.default_rng(bits + 100)
    T = 259
    codes = rng.integers(0, 1 << bits, size=(T, 2048))
    sb = rng.integers(0, 0x7C00, size=(T, 16)).astype(np.uint16)
    sb[:, :3] = [0, 1, 0x7BFF]
    zp = rng.integers(0, 1 << bits, size=(T, 16))
    zp[:, :2] = [0, (1 << bits) - 1]
    packed = P.asym_pack(bits, codes, sb, zp)
    log(f"asym decode arbitrary {fmt} {dtype}")
    y = qa.qr_decode(fmt, dev(packed), T * 2048, DT[dtype])
    torch.cuda.synchronize()
    assert np.array_equal(u16(y), oracle.decode(BITS[fmt], dtype, packed, T * 2048))


@pytest.mark.parametrize("fmt", AFMTS)
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 15, 16])
@pytest.mark.parametrize("ntiles", [3, 133])
def test_asym_reduce_parity(qa, oracle, fmt, dtype, R, ntiles):
    fid = BITS[fmt]
    n = ntiles * 2048
    kinds = ["normal", "groups", "scales", "outliers"]
    xs = [agen(kinds[r % 4], dtype, n, seed=2000 * R + 10 * r + ntiles) for r in range(R)]
    log(f"asym reduce {fmt} {dtype} R={R} tiles={ntiles}")
    packed = [qa.qr_encode(fmt, dev(x, DT[dtype])) for x in xs]
    out, y = qa.qr_reduce_compressed(fmt, DT[dtype], packed, n)
    out2, none = qa.qr_reduce_compressed(fmt, DT[dtype], packed, n, with_output=False)
    torch.cuda.synchronize()
    assert none is None
    wranks = [oracle.encode(fid, dtype, x) for x in xs]
    for r in range(R):
        assert np.array_equal(packed[r].cpu().numpy(), wranks[r]), r
    wout, wy = oracle.reduce(fid, dtype, wranks, n)
    got = out.cpu().numpy()
    assert np.array_equal(got, wout), f"re-encoded tiles differ at {first_diff(got, wout)}"
    assert np.array_equal(u16(y), wy)
    assert np.array_equal(out2.cpu().numpy(), wout)


@pytest.mark.parametrize("fi,fo", [("asym4", "asym8"), ("asym8", "asym4")])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("R", [1, 4, 8, 16])
def test_asym_reduce_mixed_parity(qa, oracle, fi, fo, dtype, R):
    n = 37 * 2048
    kinds = ["normal", "groups", "scales", "outliers"]
    xs = [agen(kinds[r % 4], dtype, n, seed=91 * R + r) for r in range(R)]
    log(f"asym reduce mixed {fi}->{fo} {dtype} R={R}")
    packed = [qa.qr_encode(fi, dev(x, DT[dtype])) for x in xs]
    out, y = qa.qr_reduce_compressed_mixed(fi, fo, DT[dtype], packed, n)
    torch.cuda.synchronize()
    assert out.numel() == oracle.packed_bytes(BITS[fo], n)
    wout, wy = oracle.reduce_mixed(BITS[fi], BITS[fo], dtype,
                                   [oracle.encode(BITS[fi], dtype, x) for x in xs], n)
    assert np.array_equal(out.cpu().numpy(), wout)
    assert np.array_equal(u16(y), wy)


def test_asym_hand_built_groups(qa, oracle):
    """Groups whose parameters are known by hand: the fp16 subnormal range that
    clamps the zero point, the bf16 range that saturates the scale, and the
    group minimum and maximum held by different lanes."""
    for fmt, bits in (("asym4", 4), ("asym8", 8)):
        qmax = (1 << bits) - 1
        k = 22 if bits == 4 else 357
        x16 = np.zeros(2048)
        x16[0] = -k * 2.0 ** -24                 # group 0: z clamps to qmax, scale 2^-24
        x16[128 + 5], x16[128 + 100] = -3.0, 5.0  # group 1: min in lane 4, max in lane 7
        xb16 = P.f16_bits(x16)
        xbf = np.zeros(2048)
        xbf[0] = -2.0 ** 30                      # group 0: scale saturates at 65504, z = qmax
        xbbf = P.bf16_bits(xbf)
        log(f"asym hand-built groups {fmt}")
        for dtype, xb, want_sb in (("fp16", xb16, 0x0001), ("bf16", xbbf, 0x7BFF)):
            p = qa.qr_encode(fmt, dev(xb, DT[dtype]))
            torch.cuda.synchronize()
            got = p.cpu().numpy()
            codes, sb, zp = P.asym_unpack(bits, got)
            assert sb[0, 0] == want_sb and zp[0, 0] == qmax, (fmt, dtype)
            assert np.array_equal(got, oracle.encode(BITS[fmt], dtype, xb)), (fmt, dtype)


# ---------------------------------------------------------------------------
# FP4 E2M1 block codec (hardware conversions)
# ---------------------------------------------------------------------------

def gen_fp4(kind, dtype, n, seed):
    """Value families for FP4: the common ones, plus blocks on the E2M1 grid
    (v * s with a 6 * s anchor) and blocks of midpoints between E2M1 values
    (ties at every spacing)."""
    if kind not in ("grid", "ties"):
        return gen(kind, dtype, n, seed)
    rng = np.random.default_rng(seed)
    nb = n // 32
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    if kind == "grid":
        v = mags[rng.integers(0, 8, size=(nb, 32))]
    else:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        v = mids[rng.integers(0, 7, size=(nb, 32))]
    v = v * np.where(rng.random((nb, 32)) < 0.5, -1.0, 1.0)
    v[:, 0] = 6.0
    x = (v * 2.0 ** rng.integers(-12, 8, size=(nb, 1))).ravel()
    if dtype == "fp16":
        return P.f16_bits(np.clip(x, -65504, 65504))
    return P.bf16_bits(x.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ntiles", [1, 5, 37, 1031])
@pytest.mark.parametrize("kind", ["normal", "outliers", "scales", "specials", "grid", "ties"])
def test_fp4_encode_decode_parity(qa, oracle, dtype, ntiles, kind):
    n = ntiles * 2048
    xb = gen_fp4(kind, dtype, n, seed=ntiles * 17 + len(kind))
    log(f"fp4 encode/decode {dtype} tiles={ntiles} {kind}")
    p = qa.qr_encode("fp4", dev(xb, DT[dtype]))
    y = qa.qr_decode("fp4", p, n, DT[dtype])
    torch.cuda.synchronize()
    want_p = oracle.encode(36, dtype, xb)
    got_p = p.cpu().numpy()
    assert np.array_equal(got_p, want_p), f"packed bytes differ at {first_diff(got_p, want_p)}"
    assert np.array_equal(u16(y), oracle.decode(36, dtype, want_p, n))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp4_decode_arbitrary_packed(qa, oracle, dtype):
    """Every code with every finite fp16 scale class (zero, subnormal, largest)."""
    rng = np.random.default_rng(36)
    T = 517
    codes = rng.integers(0, 16, size=(T, 2048))
    sb = rng.integers(0, 0x7C00, size=(T, 64)).astype(np.uint16)
    sb[:, :3] = [0, 1, 0x7BFF]
    packed = P.pack(4, codes, sb)
    log(f"fp4 decode arbitrary {dtype}")
    y = qa.qr_decode("fp4", dev(packed), T * 2048, DT[dtype])
    torch.cuda.synchronize()
    assert np.array_equal(u16(y), oracle.decode(36, dtype, packed, T * 2048))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("ntiles", [3, 133])
def test_fp4_reduce_parity(qa, oracle, dtype, R, ntiles):
    n = ntiles * 2048
    kinds = ["normal", "grid", "scales", "ties", "outliers", "specials"]
    xs = [gen_fp4(kinds[r % 6], dtype, n, seed=3000 * R + 10 * r + ntiles) for r in range(R)]
    log(f"fp4 reduce {dtype} R={R} tiles={ntiles}")
    packed = [qa.qr_encode("fp4", dev(x, DT[dtype])) for x in xs]
    out, y = qa.qr_reduce_compressed("fp4", DT[dtype], packed, n)
    out2, none = qa.qr_reduce_compressed("fp4", DT[dtype], packed, n, with_output=False)
    torch.cuda.synchronize()
    assert none is None
    wranks = [oracle.encode(36, dtype, x) for x in xs]
    for r in range(R):
        assert np.array_equal(packed[r].cpu().numpy(), wranks[r]), r
    wout, wy = oracle.reduce(36, dtype, wranks, n)
    got = out.cpu().numpy()
    assert np.array_equal(got, wout), f"re-encoded tiles differ at {first_diff(got, wout)}"
    assert np.array_equal(u16(y), wy)
    assert np.array_equal(out2.cpu().numpy(), wout)


def test_fp4_reduce_fp16_overflow(qa, oracle):
    """fp16 sums that overflow to +-inf: scale saturates at 65504, codes +-6."""
    n = 2 * 2048
    xb = [P.f16_bits(np.full(n, 60000.0)) for r in range(3)]
    xb[1][::3] = P.f16_bits(-60000.0)
    log("fp4 reduce fp16 overflow")
    packed = [qa.qr_encode("fp4", dev(x, torch.float16)) for x in xb]
    out, y = qa.qr_reduce_compressed("fp4", torch.float16, packed, n)
    torch.cuda.synchronize()
    wout, wy = oracle.reduce(36, "fp16", [oracle.encode(36, "fp16", x) for x in xb], n)
    assert np.array_equal(out.cpu().numpy(), wout) and np.array_equal(u16(y), wy)


def test_graph_replay_matches_eager(qa):
    """A step (R encodes + the fused reduce) captured in a HIP graph and
    replayed three times, with eager work and synchronizations in between:
    every replay rewrites the outputs (cleared with an eager fill before it)
    with exactly the bytes of the eager step."""
    w = W.small(W.WORKLOADS["int4_r8_fp16_32x1024x4096"], 16 * 2048 * 4)
    xs = [x.cuda() for x in W.inputs(w, seed=5)]
    packed = [torch.empty(qa.qr_packed_bytes("int4", w.n), dtype=torch.uint8, device="cuda") for _ in xs]
    out = torch.empty(qa.qr_packed_bytes("int4", w.n), dtype=torch.uint8, device="cuda")
    y = torch.empty(w.n, dtype=w.dtype, device="cuda")

    def step():
        for x, p in zip(xs, packed):
            qa.qr_encode("int4", x, p)
        qa.qr_reduce_compressed("int4", w.dtype, packed, w.n, packed_out=out, y_out=y)

    log("graph replay vs eager")
    step()
    torch.cuda.synchronize()
    want = [p.clone() for p in packed] + [out.clone(), y.view(torch.int16).clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in packed + [out]:
            t.fill_(0xA5)
        y.fill_(-1.0)
        other = qa.qr_encode("int8", xs[rep])   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [p.clone() for p in packed] + [out.clone(), y.view(torch.int16).clone()]
        assert all(torch.equal(a, b) for a, b in zip(got, want)), rep
        del other


# ---------------------------------------------------------------------------
# grid-stride loops: the library built with its grid capped at 3 workgroups
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_grid():
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_helpers", "libqr_smallgrid.so")
    L = ctypes.CDLL(path)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.qr_packed_bytes.restype = sz
    L.qr_packed_bytes.argtypes = [i, sz]
    L.qr_encode.argtypes = [i, i, vp, vp, sz, vp]
    L.qr_decode.argtypes = [i, i, vp, vp, sz, vp]
    L.qr_reduce_compressed.argtypes = [i, i, ctypes.POINTER(vp), i, vp, vp, sz, vp]
    return L


@pytest.mark.parametrize("fmt", ["int3", "int4", "int8", "asym4", "asym8", "fp4"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_grid_stride_loops(small_grid, oracle, fmt, dtype):
    """With 3 workgroups (12 waves) every wave loops over many tiles, and the
    encode prefetches each next tile while it encodes the current one: encode,
    decode and the reduce (R = 3, with and without y) against the oracle, on
    a tile count that the 12 waves do not divide."""
    import ctypes
    L = small_grid
    fid, dt = BITS[fmt], (0 if dtype == "fp16" else 1)
    ntiles = 151
    n = ntiles * 2048
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    kinds = ["normal", "scales", "specials"]
    xs = [gen(kinds[r], dtype, n, seed=500 + 10 * r + fid) for r in range(3)]
    log(f"grid-stride loops {fmt} {dtype} tiles={ntiles}")
    pb = L.qr_packed_bytes(fid, n)
    xd = [dev(x, DT[dtype]) for x in xs]
    packed = [torch.empty(pb, dtype=torch.uint8, device="cuda") for _ in xs]
    for x, p in zip(xd, packed):
        assert L.qr_encode(fid, dt, x.data_ptr(), p.data_ptr(), n, st) == 0
    y = torch.empty(n, dtype=DT[dtype], device="cuda")
    assert L.qr_decode(fid, dt, packed[0].data_ptr(), y.data_ptr(), n, st) == 0
    out = torch.empty(pb, dtype=torch.uint8, device="cuda")
    out2 = torch.empty(pb, dtype=torch.uint8, device="cuda")
    yr = torch.empty(n, dtype=DT[dtype], device="cuda")
    arr = (ctypes.c_void_p * 3)(*[p.data_ptr() for p in packed])
    assert L.qr_reduce_compressed(fid, dt, arr, 3, out.data_ptr(), yr.data_ptr(), n, st) == 0
    assert L.qr_reduce_compressed(fid, dt, arr, 3, out2.data_ptr(), None, n, st) == 0
    torch.cuda.synchronize()
    wr = [oracle.encode(fid, dtype, x) for x in xs]
    for r in range(3):
        assert np.array_equal(packed[r].cpu().numpy(), wr[r]), r
    assert np.array_equal(u16(y), oracle.decode(fid, dtype, wr[0], n))
    wout, wy = oracle.reduce(fid, dtype, wr, n)
    assert np.array_equal(out.cpu().numpy(), wout) and np.array_equal(out2.cpu().numpy(), wout)
    assert np.array_equal(u16(yr), wy)


@pytest.mark.parametrize("fmt", ["int3", "int4", "int8", "asym4", "asym8", "fp4"])
def test_buffers_at_16_byte_offsets(qa, oracle, fmt):
    """Every buffer (inputs, packed ranks, packed output, y) starts 16 bytes
    into its allocation, so no tile is aligned beyond the documented 16
    bytes: encode, decode and the R = 3 reduce still match the oracle."""
    fid = BITS[fmt]
    ntiles = 21
    n = ntiles * 2048
    pb = qa.qr_packed_bytes(fmt, n)
    xs = [gen(k, "bf16", n, seed=900 + i) for i, k in enumerate(("normal", "scales", "outliers"))]
    log(f"16-byte offsets {fmt}")

    def at16(numel, dtype):
        return torch.empty(numel + 16 // torch.tensor([], dtype=dtype).element_size(), dtype=dtype,
                           device="cuda")[16 // torch.tensor([], dtype=dtype).element_size():]

    xd = []
    for x in xs:
        t = at16(n, torch.bfloat16)
        t.copy_(dev(x, torch.bfloat16))
        xd.append(t)
    packed = [at16(pb, torch.uint8) for _ in xs]
    assert all(p.data_ptr() % 256 == 16 for p in packed)
    for x, p in zip(xd, packed):
        qa.qr_encode(fmt, x, p)
    y = at16(n, torch.bfloat16)
    qa.qr_decode(fmt, packed[1], n, torch.bfloat16, y=y)
    out, yr = at16(pb, torch.uint8), at16(n, torch.bfloat16)
    qa.qr_reduce_compressed(fmt, torch.bfloat16, packed, n, packed_out=out, y_out=yr)
    torch.cuda.synchronize()
    wr = [oracle.encode(fid, "bf16", x) for x in xs]
    for r in range(3):
        assert np.array_equal(packed[r].cpu().numpy(), wr[r]), r
    assert np.array_equal(u16(y), oracle.decode(fid, "bf16", wr[1], n))
    wout, wy = oracle.reduce(fid, "bf16", wr, n)
    assert np.array_equal(out.cpu().numpy(), wout)
    assert np.array_equal(u16(yr), wy)


def test_binding_rejects_short_or_mistyped_tensors(qa):
    """The binding checks tensor byte sizes, the output dtype and the device
    before calling the library (the C ABI takes raw pointers and cannot)."""
    n = 4 * 2048
    x = torch.zeros(n, dtype=torch.float16, device="cuda")
    p = qa.qr_encode("int4", x)
    with pytest.raises(ValueError):
        qa.qr_encode("int4", x, torch.empty(4 * 1152 - 1, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        qa.qr_decode("int4", p, n, torch.float16, y=torch.empty(n - 1, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        qa.qr_decode("int4", p, n, torch.float16, y=torch.empty(n, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        qa.qr_decode("int4", p[:100], n, torch.float16)
    with pytest.raises(ValueError):
        qa.qr_reduce_compressed("int4", torch.float16, [p, p[:-16]], n)
    with pytest.raises(ValueError):
        qa.qr_reduce_compressed_mixed("int4", "int8", torch.float16, [p], n,
                                      packed_out=torch.empty(4 * 1152, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        qa.qr_encode("int5", x)
    torch.cuda.synchronize()


def test_asym_group_params_device_function(oracle):
    """The library's asymmetric group parameters (scale bits, multiplier, zero
    point) against the oracle's, for every positive finite fp16 h as the
    ranges [0, h], [-h, 0] and [-h, h], 100,000 random fp16 ranges, bf16
    ranges that saturate the scale or overflow hi - lo, and ranges with
    infinite ends (fp16 sums that overflowed)."""
    import ctypes
    import os
    lib = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_helpers", "libscale_check.so")
    L = ctypes.CDLL(lib)
    L.qr_test_group_params.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int]
    h = P.f16_value(np.arange(1, 0x7C00, dtype=np.uint16)).astype(np.float64)
    rng = np.random.default_rng(77)
    fin = P.f16_value(rng.integers(0, 0x7C00, size=(100000, 2)).astype(np.uint16)).astype(np.float64)
    big = P.bf16_value(rng.integers(0x4700, 0x7F80, size=(2000, 2)).astype(np.uint16)).astype(np.float64)
    inf = np.inf
    lo = np.concatenate([np.zeros_like(h), -h, -h, -fin[:, 0], -big[:, 0], [-inf, 0.0, -inf, -0.0, 0.0, -1.0]])
    hi = np.concatenate([h, np.zeros_like(h), h, fin[:, 1], big[:, 1], [0.0, inf, inf, 0.0, 0.0, inf]])
    n = lo.size
    lo_d = torch.tensor(lo, dtype=torch.float32, device="cuda")
    hi_d = torch.tensor(hi, dtype=torch.float32, device="cuda")
    log(f"asym group params on {n} ranges")
    for bits, fid in ((4, 20), (8, 24)):
        d = torch.zeros(n, dtype=torch.int32, device="cuda")
        e = torch.zeros(n, dtype=torch.float32, device="cuda")
        z = torch.zeros(n, dtype=torch.int32, device="cuda")
        assert L.qr_test_group_params(fid, lo_d.data_ptr(), hi_d.data_ptr(), d.data_ptr(), e.data_ptr(),
                                      z.data_ptr(), n) == 0
        gd, ge, gz = d.cpu().numpy(), e.cpu().numpy(), z.cpu().numpy()
        lo32, hi32 = lo.astype(np.float32), hi.astype(np.float32)
        bad = []
        for i in range(n):
            wd, we, wz = oracle.group_params(bits, float(lo32[i]), float(hi32[i]))
            if gd[i] != wd or gz[i] != wz or np.float32(ge[i]).tobytes() != np.float32(we).tobytes():
                bad.append((float(lo32[i]), float(hi32[i]), hex(gd[i]), hex(wd), gz[i], wz))
                if len(bad) > 5:
                    break
        assert not bad, (bits, bad)


def test_c_abi_from_plain_c():
    """tests/c_abi/abi_check.c, built with gcc against include/qr.h and
    libqr.so, runs as a child process: exact round trips and exact two-rank
    reductions for INT3/INT4/INT8 in fp16 and bf16, and rejected arguments."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_check")
    log("plain C use of the ABI")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks hold" in res.stdout


def test_calls_on_a_side_stream(qa, oracle):
    """Every entry point enqueues on the stream it is given: the whole path on
    a separately created stream (default priority), synchronized through that
    stream alone, matches the oracle."""
    n = 9 * 2048
    xs = [gen("normal", "fp16", n, seed=40 + r) for r in range(3)]
    side = torch.cuda.Stream()
    xd = [dev(x, torch.float16) for x in xs]
    torch.cuda.synchronize()
    log("side stream")
    with torch.cuda.stream(side):
        packed = [torch.empty(qa.qr_packed_bytes("int3", n), dtype=torch.uint8, device="cuda") for _ in xs]
        out = torch.empty(qa.qr_packed_bytes("int3", n), dtype=torch.uint8, device="cuda")
        y = torch.empty(n, dtype=torch.float16, device="cuda")
        yd = torch.empty(n, dtype=torch.float16, device="cuda")
    for x, p in zip(xd, packed):
        qa.qr_encode("int3", x, p, stream=side)
    qa.qr_reduce_compressed("int3", torch.float16, packed, n, packed_out=out, y_out=y, stream=side)
    qa.qr_decode("int3", out, n, torch.float16, y=yd, stream=side)
    side.synchronize()
    wr = [oracle.encode(3, "fp16", x) for x in xs]
    wout, wy = oracle.reduce(3, "fp16", wr, n)
    assert np.array_equal(out.cpu().numpy(), wout)
    assert np.array_equal(u16(y), wy) and np.array_equal(u16(yd), wy)


def test_concurrent_host_threads(qa, oracle):
    """The library keeps no state between calls: four host threads, each with
    its own stream (default priority) and format, run encode -> reduce ->
    decode 20 times at once (ctypes releases the GIL around each call, so the
    C calls overlap).  Every thread's result matches the oracle."""
    import threading

    n, R, iters = 37 * 2048, 3, 20
    cases = [("int3", "fp16"), ("int4", "bf16"), ("int8", "fp16"), ("fp4", "bf16")]
    bufs = []
    for k, (fmt, dt) in enumerate(cases):
        xs = [gen("outliers", dt, n, seed=200 + 10 * k + r) for r in range(R)]
        pb = qa.qr_packed_bytes(fmt, n)
        bufs.append({
            "host": xs,
            "x": [dev(x, DT[dt]) for x in xs],
            "packed": [torch.empty(pb, dtype=torch.uint8, device="cuda") for _ in range(R)],
            "out": torch.empty(pb, dtype=torch.uint8, device="cuda"),
            "y": torch.empty(n, dtype=DT[dt], device="cuda"),
            "yd": torch.empty(n, dtype=DT[dt], device="cuda"),
            "stream": torch.cuda.Stream(),
        })
    torch.cuda.synchronize()
    errors = []

    def work(k):
        fmt, dt = cases[k]
        b = bufs[k]
        try:
            for _ in range(iters):
                for x, p in zip(b["x"], b["packed"]):
                    qa.qr_encode(fmt, x, p, stream=b["stream"])
                qa.qr_reduce_compressed(fmt, DT[dt], b["packed"], n, packed_out=b["out"], y_out=b["y"],
                                        stream=b["stream"])
                qa.qr_decode(fmt, b["out"], n, DT[dt], y=b["yd"], stream=b["stream"])
        except Exception as e:   # reported by the main thread
            errors.append((fmt, e))

    log("concurrent host threads")
    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for b in bufs:
        b["stream"].synchronize()
    assert not errors, errors
    for (fmt, dt), b in zip(cases, bufs):
        wr = [oracle.encode(BITS[fmt], dt, x) for x in b["host"]]
        wout, wy = oracle.reduce(BITS[fmt], dt, wr, n)
        for p, w in zip(b["packed"], wr):
            assert np.array_equal(p.cpu().numpy(), w), fmt
        assert np.array_equal(b["out"].cpu().numpy(), wout), fmt
        assert np.array_equal(u16(b["y"]), wy) and np.array_equal(u16(b["yd"]), wy), fmt


@pytest.mark.parametrize("fmt", FMTS + AFMTS + ("fp4",))
def test_repeat_runs_are_bit_identical(qa, fmt):
    """Determinism control: the same inputs through every entry point twice,
    at a size with many more tiles than the chip has waves in flight, give
    byte-identical outputs (no order-dependent arithmetic, no stale LDS)."""
    n = 3000 * 2048
    R = 5
    xs = [dev(gen("outliers", "bf16", n, seed=60 + r), torch.bfloat16) for r in range(R)]
    log(f"determinism {fmt}")
    runs = []
    for _ in range(2):
        packed = [qa.qr_encode(fmt, x) for x in xs]
        out, y = qa.qr_reduce_compressed(fmt, torch.bfloat16, packed, n)
        yd = qa.qr_decode(fmt, out, n, torch.bfloat16)
        torch.cuda.synchronize()
        runs.append([p.cpu() for p in packed] + [out.cpu(), y.view(torch.int16).cpu(),
                                                 yd.view(torch.int16).cpu()])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_earlier_unrelated_hip_error_is_not_reported(qa, oracle):
    """A call returns the status of its own launch: an error that an earlier,
    unrelated HIP call left on the thread (here a host-side invalid device
    number, no GPU work involved) does not fail the call."""
    import ctypes

    n = 4 * 2048
    xb = gen("normal", "fp16", n, seed=5)
    x = dev(xb, torch.float16)
    packed = torch.empty(qa.qr_packed_bytes("int4", n), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already loaded in this process
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipGetLastError.restype = ctypes.c_int
    log("stale HIP error")
    assert hip.hipSetDevice(1 << 20) != 0
    try:
        qa.qr_encode("int4", x, packed)
    finally:
        hip.hipGetLastError()   # clear it before torch's next launch check
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle.encode(4, "fp16", xb))


@pytest.mark.parametrize("fmt", ["int3", "int8", "asym8", "fp4"])
def test_buffers_beyond_4_gib(qa, oracle, fmt):
    """Byte offsets past 2^32: two ranks of 2,050,131 tiles (4,198,668,288
    bf16 values, 8.4 GB each, a count that is not a multiple of the four
    tiles of a workgroup), so that the inputs and outputs, and the packed
    buffers of the 8-bit formats, extend past 4 GiB.  The encode, the fused
    reduce and the standalone decode are compared with the oracle on sampled
    tiles, among them the tiles next to the 4 GiB mark of each buffer."""
    ntiles = 2_050_131
    n = ntiles * 2048
    fid = BITS[fmt]
    tb = oracle.packed_bytes(fid, 2048)
    log(f"beyond 4 GiB {fmt} n={n}")
    g = torch.Generator(device="cuda").manual_seed(11)
    xs = [torch.randn(n, dtype=torch.bfloat16, device="cuda", generator=g) for _ in range(2)]
    packed = [qa.qr_encode(fmt, x) for x in xs]
    out, y = qa.qr_reduce_compressed(fmt, torch.bfloat16, packed, n)
    yd = qa.qr_decode(fmt, out, n, torch.bfloat16)
    torch.cuda.synchronize()
    edge = {(1 << 32) // 4096 - 1, (1 << 32) // 4096, (1 << 32) // tb, (1 << 32) // tb + 1}
    rng = np.random.default_rng(3)
    tiles = sorted(t for t in edge | {0, ntiles - 1} | set(rng.integers(0, ntiles, 24).tolist())
                   if t < ntiles)
    for t in tiles:
        xv = [u16(x[t * 2048:(t + 1) * 2048]) for x in xs]
        pv = [p[t * tb:(t + 1) * tb].cpu().numpy() for p in packed]
        for r in range(2):
            assert np.array_equal(pv[r], oracle.encode(fid, "bf16", xv[r])), (fmt, t, r)
        wout, wy = oracle.reduce(fid, "bf16", pv, 2048)
        assert np.array_equal(out[t * tb:(t + 1) * tb].cpu().numpy(), wout), (fmt, t)
        assert np.array_equal(u16(y[t * 2048:(t + 1) * 2048]), wy), (fmt, t)
        assert np.array_equal(u16(yd[t * 2048:(t + 1) * 2048]), wy), (fmt, t)
    del xs, packed, out, y, yd
    torch.cuda.empty_cache()


FAMILIES = {"int": ("int3", "int4", "int8"), "asym": ("asym4", "asym8"), "fp4": ("fp4",)}


@pytest.mark.parametrize("block", range(6))
def test_random_cases_match_oracle(qa, oracle, block):
    """Seeded random cases across the whole surface: a format family, an input
    and an output format within it, the dtype, R in [1, 16], a tile count in
    [1, 300], and per rank one of the value families of the oracle's model
    cross-check (heavy tails, blocks over the dtype's whole exponent range,
    exact rounding ties for every format, zero / single / saturating /
    subnormal blocks).  Encode, the fused reduce and the decode of its output
    are compared with the oracle byte for byte."""
    import test_oracle_model as TM

    for case in range(20):
        seed = 1000 * block + case
        rng = np.random.default_rng(seed)
        fam = FAMILIES[("int", "asym", "fp4")[rng.integers(3)]]
        fi, fo = fam[rng.integers(len(fam))], fam[rng.integers(len(fam))]
        dtype = ("fp16", "bf16")[rng.integers(2)]
        R = int(rng.integers(1, 17))
        ntiles = int(rng.integers(1, 301))
        n = ntiles * 2048
        kinds = [TM.FAMILIES[rng.integers(len(TM.FAMILIES))] for _ in range(R)]
        log(f"random case seed={seed}: {fi}->{fo} {dtype} R={R} tiles={ntiles} {kinds}")
        xs = [TM.family(k, dtype, rng, tiles=ntiles) for k in kinds]
        packed = [qa.qr_encode(fi, dev(x, DT[dtype])) for x in xs]
        out, y = qa.qr_reduce_compressed_mixed(fi, fo, DT[dtype], packed, n)
        yd = qa.qr_decode(fo, out, n, DT[dtype])
        torch.cuda.synchronize()
        wr = [oracle.encode(BITS[fi], dtype, x) for x in xs]
        for r in range(R):
            assert np.array_equal(packed[r].cpu().numpy(), wr[r]), (seed, "encode", r)
        wout, wy = oracle.reduce_mixed(BITS[fi], BITS[fo], dtype, wr, n)
        assert np.array_equal(out.cpu().numpy(), wout), (seed, "packed_out")
        assert np.array_equal(u16(y), wy), (seed, "y_out")
        assert np.array_equal(u16(yd), oracle.decode(BITS[fo], dtype, wout, n)), (seed, "decode")
