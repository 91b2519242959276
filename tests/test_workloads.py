"""The seeded input generator: shapes, determinism and distributions."""
import math

import torch

import workloads as W


def test_catalogue():
    w = W.WORKLOADS
    assert w["int3_r2_fp16_8k"].n == 8192 and w["int3_r2_fp16_8k"].ranks == 2
    assert w["int3_bf16_codec_8m"].n == 8388608 and not w["int3_bf16_codec_8m"].reduce
    assert w["int3_r8_bf16_1024x8192"].n == 1024 * 8192 and w["int3_r8_bf16_1024x8192"].ranks == 8
    assert w["int4_r8_fp16_32x1024x4096"].n == 134217728
    assert w["sweep_r4_fp16_int8_512mib"].n == 268435456
    # the codec workload's input is rank 0's input of the INT4 R=8 workload
    c, b = W.small(w["int4_fp16_codec_32x1024x4096"], 4096 * 4), W.small(w["int4_r8_fp16_32x1024x4096"], 4096 * 4)
    assert not c.reduce and c.ranks == 1
    assert torch.equal(W.rank_input(c, 0, seed=1).view(torch.int16), W.rank_input(b, 0, seed=1).view(torch.int16))
    # INT3 and INT4 over two ranks see the same inputs
    a, b = W.small(w["int3_r2_fp16_32x1024x4096"], 4096 * 4), W.small(w["int4_r2_fp16_32x1024x4096"], 4096 * 4)
    for r in range(2):
        assert torch.equal(W.rank_input(a, r, seed=2).view(torch.int16), W.rank_input(b, r, seed=2).view(torch.int16))
    for v in w.values():
        assert v.n % 2048 == 0


def test_deterministic_and_distinct():
    w = W.small(W.WORKLOADS["int3_r8_bf16_1024x8192"], 1 << 16)
    a = W.rank_input(w, 0, seed=1)
    b = W.rank_input(w, 0, seed=1)
    c = W.rank_input(w, 1, seed=1)
    d = W.rank_input(w, 0, seed=2)
    assert a.dtype == torch.bfloat16 and a.numel() == 1 << 16
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a, c) and not torch.equal(a, d)


def test_distributions():
    w = W.small(W.WORKLOADS["int3_r8_bf16_1024x8192"], 1 << 20)
    x = W.rank_input(w, 0).float()
    big = x.abs() > 5
    assert 0.0005 < big.float().mean() < 0.0015          # 0.1% outliers x50
    assert abs(x[~big].std().item() - 0.5) < 0.01
    w5 = W.small(W.WORKLOADS["int4_r8_fp16_32x1024x4096"], 4096 * 256)
    s = W.channel_sigmas(w5, 0)
    assert s.min() >= 0.01 * 0.999 and s.max() <= 20 * 1.001
    lg = torch.log(s)
    assert abs(lg.mean().item() - (math.log(0.01) + math.log(20)) / 2) < 0.2
    x0 = W.rank_input(w5, 0).float().view(-1, 4096)
    x1 = W.rank_input(w5, 1).float().view(-1, 4096)
    r = x0.std(dim=0) / s
    assert abs(r.mean().item() - 1) < 0.02               # same channel spread on every rank
    assert not torch.equal(x0, x1)
