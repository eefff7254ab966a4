"""Seeded input generation: determinism, chunk independence, storage casts (CPU only)."""
import numpy as np
import torch

import oracle
import synthetic
from synthetic.gen import normal, quantize_fp8_blocks


def test_same_seed_same_bytes():
    a = synthetic.make_workload("tiny_decode")
    b = synthetic.make_workload("tiny_decode")
    for name in ("index_q", "index_w", "k_cache", "q", "kv", "sink"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_chunk_regeneration_matches_full_tensor():
    full = normal(123, 9, (6, 70, 128), sigma=0.5)
    part = normal(123, 9, (6, 70, 128), sigma=0.5, chunks=[4, 1])
    assert torch.equal(part[0], full[4]) and torch.equal(part[1], full[1])


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    y = x.to(torch.bfloat16).to(torch.float32)
    assert y.tolist() == [1.0, 1.0 + 2 ** -6, -1.0]


def test_fp8_block_quantiser():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(5, 7, 128, generator=g)
    x[0, 0] = 0.0
    codes, scales = quantize_fp8_blocks(x)
    assert codes.dtype == torch.uint8 and scales.shape == (5, 7)
    assert scales[0, 0] == 1.0
    vals = oracle.decode_fp8_e4m3(codes.numpy())
    assert np.abs(vals).max() <= 448.0
    # the block maximum maps to +-448 (amax / 448 scaling)
    amax_code = np.abs(vals).max(axis=-1)
    assert np.all(amax_code.ravel()[1:] == 448.0) and amax_code[0, 0] == 0.0
    deq = vals * scales.numpy()[..., None]
    rel = np.abs(deq - x.numpy()) / np.maximum(np.abs(x.numpy()), 1e-3)
    assert np.median(rel) < 0.04  # 3 mantissa bits


def test_workload_shapes_scaled():
    w = synthetic.make_workload("full_decode_step", B=2, S_max=512, Hq=16, Dqk=64, Dv=32, window=8, topk=16)
    assert w.index_q.shape == (2, 64, 128) and w.k_cache.shape == (2, 512, 128)
    assert w.q.shape == (2, 1, 16, 64) and w.kv.shape == (2, 512, 64)
    assert w.positions.tolist() == [511, 511]
    w4 = synthetic.make_workload("fp8_long_decode", M=2, S_max=1000, vl_lo=500)
    assert w4.k_cache.dtype == torch.uint8 and w4.k_scale.shape == (2, 1000)
    assert all(499 <= int(p) <= 999 for p in w4.positions)
