"""Seeded synthetic inputs for the codec and the compressed-domain reduction.

Shapes, sizes and value distributions only: this module holds none of the
codec's arithmetic and is the one piece shared by the HIP path's tests and
benchmark and by the CPU oracle's checks.  Both sides always receive the very
same fp16/bf16 bytes (generated once, copied where needed).

Workloads (values per rank; "MB" read as MiB so sizes are whole 2048-value
tiles):
  int3_r2_fp16_8k          INT3, fp16, R=2, 8192 values, N(0,1)
  int3_bf16_codec_8m       INT3, bf16, encode/decode only, 8,388,608 values,
                           N(0,1) with 0.1% of entries multiplied by 50
  int3_r8_bf16_1024x8192   INT3, bf16, R=8, [1024 tokens x 8192 hidden],
                           N(0, 0.5^2) with 0.1% of entries multiplied by 50
  sweep_r4_fp16_<fmt>_<s>mib  INT3/INT4/INT8, fp16, R=4, s in {1,16,128,512} MiB
                           per rank, N(0,1)
  int4_r8_fp16_32x1024x4096  INT4, fp16, R=8, [32 x 1024 x 4096] activations
                           with per-channel spread: channel c (last dim) has
                           std sigma_c = exp(U[ln 0.01, ln 20]), drawn once per
                           seed and shared by all ranks; values sigma_c * N(0,1)
                           independent per rank.
  int6_r8_fp16_32x1024x4096  the same inputs with the re-encoded sum in INT8
                           (INT4 reduce inputs + INT8 gather payload, "INT6").
  asym4_r8_fp16_32x1024x4096  the same inputs through the asymmetric 4-bit
                           group codec (128-value groups, scale + zero point).
  asym6_r8_fp16_32x1024x4096  the same inputs, asymmetric 4-bit reduce inputs
                           and an asymmetric 8-bit re-encoded sum.
  fp4_r8_fp16_32x1024x4096  the same inputs through the FP4 E2M1 block codec.
  int4_r8_fp16_4x1024x4096  one rank's share of that reduce in the two-shot
                           scheme: R = 8 segments of n / 8 = 4 x 1024 x 4096
                           values (the same channel spread).
  int4_r8_bf16_32x1024x4096  the [32 x 1024 x 4096] INT4 R=8 workload with bf16
                           activations (same channel spread, its own streams).
  int3_r2_fp16_32x1024x4096  INT3 over R=2 ranks of the same shape and spread
                           (tensor parallelism 2, where the pages recommend INT3).
  int4_r2_fp16_32x1024x4096  INT4 on the same two ranks' inputs (INT3 against
                           INT4 at tensor parallelism 2, same data).
  int4_fp16_codec_32x1024x4096  encode + decode only of rank 0's input of the
                           [32 x 1024 x 4096] INT4 workload (the receive side's
                           decode of gathered tiles, at full size).
  int3_fp16_codec_32x1024x4096  the same for INT3, on rank 0's input of the
                           INT3 two-rank workload.

Random numbers come from torch's seeded generators (Philox on the GPU, the CPU
generator on the host); each (seed, workload, rank) gets its own stream seed.
"""
import dataclasses
import math

import torch

MIB = 1 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str                 # "int3" | "int4" | "int8" | "asym4" | "asym8" | "fp4"
    dtype: torch.dtype       # torch.float16 | torch.bfloat16
    ranks: int               # R simulated rank buffers (1 = encode/decode only)
    n: int                   # values per rank
    shape: tuple             # logical shape of one rank's activation
    sigma: float = 1.0
    outlier_p: float = 0.0
    outlier_mult: float = 50.0
    channel_sigma: tuple = None   # (lo, hi) of the log-uniform channel std, or None
    reduce: bool = True
    fmt_out: str = None           # format of the re-encoded sum, if it differs from fmt
    data_key: str = None          # name whose random streams the inputs use (default: name)

    @property
    def out_fmt(self):
        return self.fmt_out or self.fmt

    @property
    def io_dtype(self):
        return "fp16" if self.dtype == torch.float16 else "bf16"


def _sweep():
    out = {}
    for fmt in ("int3", "int4", "int8"):
        for mib in (1, 16, 128, 512):
            n = mib * MIB // 2
            name = f"sweep_r4_fp16_{fmt}_{mib}mib"
            out[name] = Workload(name, fmt, torch.float16, 4, n, (n,))
    return out


WORKLOADS = {
    "int3_r2_fp16_8k": Workload("int3_r2_fp16_8k", "int3", torch.float16, 2, 8192, (8192,)),
    "int3_bf16_codec_8m": Workload("int3_bf16_codec_8m", "int3", torch.bfloat16, 1, 8 * MIB, (8 * MIB,),
                                   outlier_p=0.001, reduce=False),
    "int3_r8_bf16_1024x8192": Workload("int3_r8_bf16_1024x8192", "int3", torch.bfloat16, 8, 1024 * 8192,
                                       (1024, 8192), sigma=0.5, outlier_p=0.001),
    **_sweep(),
    "int4_r8_fp16_32x1024x4096": Workload("int4_r8_fp16_32x1024x4096", "int4", torch.float16, 8,
                                          32 * 1024 * 4096, (32, 1024, 4096),
                                          channel_sigma=(0.01, 20.0)),
    # mixed formats per phase ("INT6"): INT4 reduce inputs, INT8 re-encoded sum
    "int6_r8_fp16_32x1024x4096": Workload("int6_r8_fp16_32x1024x4096", "int4", torch.float16, 8,
                                          32 * 1024 * 4096, (32, 1024, 4096),
                                          channel_sigma=(0.01, 20.0), fmt_out="int8",
                                          data_key="int4_r8_fp16_32x1024x4096"),
    # asymmetric group codec on the same activations
    "asym4_r8_fp16_32x1024x4096": Workload("asym4_r8_fp16_32x1024x4096", "asym4", torch.float16, 8,
                                           32 * 1024 * 4096, (32, 1024, 4096),
                                           channel_sigma=(0.01, 20.0),
                                           data_key="int4_r8_fp16_32x1024x4096"),
    "asym6_r8_fp16_32x1024x4096": Workload("asym6_r8_fp16_32x1024x4096", "asym4", torch.float16, 8,
                                           32 * 1024 * 4096, (32, 1024, 4096),
                                           channel_sigma=(0.01, 20.0), fmt_out="asym8",
                                           data_key="int4_r8_fp16_32x1024x4096"),
    # one rank's share (n / 8 values from each of the 8 ranks) of the reduce above
    "int4_r8_fp16_4x1024x4096": Workload("int4_r8_fp16_4x1024x4096", "int4", torch.float16, 8,
                                         4 * 1024 * 4096, (4, 1024, 4096), channel_sigma=(0.01, 20.0)),
    # FP4 E2M1 block codec on the same activations
    "fp4_r8_fp16_32x1024x4096": Workload("fp4_r8_fp16_32x1024x4096", "fp4", torch.float16, 8,
                                         32 * 1024 * 4096, (32, 1024, 4096),
                                         channel_sigma=(0.01, 20.0),
                                         data_key="int4_r8_fp16_32x1024x4096"),
    # the same shape and channel spread with bf16 activations
    "int4_r8_bf16_32x1024x4096": Workload("int4_r8_bf16_32x1024x4096", "int4", torch.bfloat16, 8,
                                          32 * 1024 * 4096, (32, 1024, 4096), channel_sigma=(0.01, 20.0)),
    # INT3 over two ranks (tensor parallelism 2, where the pages recommend INT3)
    "int3_r2_fp16_32x1024x4096": Workload("int3_r2_fp16_32x1024x4096", "int3", torch.float16, 2,
                                          32 * 1024 * 4096, (32, 1024, 4096), channel_sigma=(0.01, 20.0)),
    # INT4 on the INT3 two-rank workload's inputs
    "int4_r2_fp16_32x1024x4096": Workload("int4_r2_fp16_32x1024x4096", "int4", torch.float16, 2,
                                          32 * 1024 * 4096, (32, 1024, 4096), channel_sigma=(0.01, 20.0),
                                          data_key="int3_r2_fp16_32x1024x4096"),
    # encode + decode only, on rank 0's input of the INT4 R=8 workload
    "int4_fp16_codec_32x1024x4096": Workload("int4_fp16_codec_32x1024x4096", "int4", torch.float16, 1,
                                             32 * 1024 * 4096, (32, 1024, 4096),
                                             channel_sigma=(0.01, 20.0), reduce=False,
                                             data_key="int4_r8_fp16_32x1024x4096"),
    "int3_fp16_codec_32x1024x4096": Workload("int3_fp16_codec_32x1024x4096", "int3", torch.float16, 1,
                                             32 * 1024 * 4096, (32, 1024, 4096),
                                             channel_sigma=(0.01, 20.0), reduce=False,
                                             data_key="int3_r2_fp16_32x1024x4096"),
}

BENCH_WORKLOAD = "int4_r8_fp16_32x1024x4096"


def derive_seed(*parts):
    """63-bit stream seed from integers/strings (splitmix64 finalizer over a running hash)."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        if isinstance(p, str):
            for ch in p.encode():
                h = ((h ^ ch) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
        else:
            h = (h + (int(p) & 0xFFFFFFFFFFFFFFFF) + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h = z ^ (z >> 31)
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def channel_sigmas(w, seed, device="cpu"):
    lo, hi = w.channel_sigma
    g = _gen(device, derive_seed(seed, w.data_key or w.name, "channels"))
    u = torch.rand(w.shape[-1], generator=g, device=device, dtype=torch.float32)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def rank_input(w, rank, seed=0, device="cpu"):
    """Rank `rank`'s input: a flat tensor of w.n values of w.dtype on `device`."""
    g = _gen(device, derive_seed(seed, w.data_key or w.name, rank))
    x = torch.randn(w.n, generator=g, device=device, dtype=torch.float32)
    if w.channel_sigma is not None:
        x.view(-1, w.shape[-1]).mul_(channel_sigmas(w, seed, device))
    elif w.sigma != 1.0:
        x.mul_(w.sigma)
    if w.outlier_p > 0:
        mask = torch.rand(w.n, generator=g, device=device) < w.outlier_p
        x[mask] *= w.outlier_mult
        del mask
    return x.to(w.dtype)


def inputs(w, seed=0, device="cpu"):
    return [rank_input(w, r, seed, device) for r in range(w.ranks)]


def small(w, n):
    """The same workload with only `n` values per rank (CPU-sized checks, size
    sweeps); with per-channel spread the channel count stays when it divides n,
    else every value is its own channel."""
    if w.channel_sigma is None:
        shape = (n,)
    elif n % w.shape[-1] == 0:
        shape = (n // w.shape[-1], w.shape[-1])
    else:
        shape = (1, n)
    return dataclasses.replace(w, n=n, shape=shape)
