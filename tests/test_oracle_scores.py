"""Pins for the oracle's format decoding and indexer scores (CPU only).

Each test checks the oracle against something other than itself: hand-derived
values (tests/golden), a library's own format conversion, a special case that
reduces to a plain matrix-vector product, or an exact algebraic invariant
(Hadamard orthogonality, stated on the NKI "Sparse Attention Indexer MX
BF16Score Kernel API Reference" page, Notes).
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


# ---------------------------------------------------------------- formats

def test_bf16_decode_matches_torch():
    g = np.random.default_rng(1)
    bits = g.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    exp_field = (bits >> 7) & 0xFF
    bits = bits[exp_field != 0xFF]  # drop inf / NaN patterns
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_fp8_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)  # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_e4m3_known_codes():
    v = oracle.decode_fp8_e4m3(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8, 0x00, 0x80, 0x07], np.uint8))
    assert list(v) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0, 0.0, 0.0, 7 * 2.0 ** -9]


# ---------------------------------------------------------------- mask bound

def test_mask_bound_is_most_negative_finite_bf16():
    mb = oracle.mask_bound()
    assert _f32_bits(mb) == 0xFF7F0000
    as_bf16 = torch.tensor([mb], dtype=torch.float32).to(torch.bfloat16)
    assert torch.isfinite(as_bf16).all() and float(as_bf16) == mb
    # -FLT_MAX would round to -inf in bf16: the failure the finite bound avoids.
    assert torch.isinf(torch.tensor([-3.4028235e38]).to(torch.bfloat16)).all()


# ---------------------------------------------------------------- n_valid

@pytest.mark.parametrize("positions,valid_len,row,s_max,expected", [
    (None, -1, 0, 100, 100),
    (None, 40, 0, 100, 40),
    ([7, 9], -1, 1, 100, 10),
    ([7, 9], 5, 1, 100, 5),
    ([7, 200], -1, 1, 100, 100),
    ([-1], -1, 0, 100, 0),
    (None, 0, 0, 100, 0),
])
def test_n_valid_rules(positions, valid_len, row, s_max, expected):
    pos = None if positions is None else np.array(positions, np.int32)
    assert oracle.n_valid(pos, valid_len, row, s_max) == expected


# ---------------------------------------------------------------- scores

def _golden_scores(golden_dir):
    with open(os.path.join(golden_dir, "score_small.json")) as f:
        return json.load(f)["cases"]


def _expected(rows, mb):
    return np.array([[mb if v == "mask" else float(v) for v in row] for row in rows], np.float32)


@pytest.mark.parametrize("relu", [False, True])
def test_scores_golden(golden_dir, relu):
    mb = oracle.mask_bound()
    for case in _golden_scores(golden_dir):
        key = "expected_relu" if relu else "expected_identity"
        if key not in case:
            continue
        got = oracle.index_score(np.array(case["q"], np.float64), np.array(case["w"], np.float32),
                                 np.array(case["k"], np.float64), scale=case["scale"],
                                 positions=np.array(case["positions"], np.int32),
                                 valid_len=case["valid_len"], rows_per_seq=case["rows_per_seq"], relu=relu)
        exp = _expected(case[key], mb)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), (case["name"], got, exp)


def test_scores_bf16_inputs_equal_f64_inputs():
    """bf16 inputs decode exactly: feeding the same values as float64 gives identical scores."""
    g = np.random.default_rng(2)
    q = torch.from_numpy(g.standard_normal((3, 5, 128)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(g.standard_normal((3, 50, 128)).astype(np.float32)).to(torch.bfloat16)
    w = g.standard_normal((3, 5)).astype(np.float32)
    pos = np.array([10, 49, 0], np.int32)
    a = oracle.index_score(q, w, k, scale=0.1, positions=pos)
    b = oracle.index_score(q.to(torch.float64), w, k.to(torch.float64), scale=0.1, positions=pos)
    assert np.array_equal(a, b)


def test_scores_single_head_is_matvec():
    """H = 1, w = 1, scale = 1: the score row is K @ q (a library mat-vec), rounded to fp32."""
    g = np.random.default_rng(3)
    q = g.standard_normal((2, 1, 128))
    k = g.standard_normal((2, 300, 128))
    got = oracle.index_score(q, np.ones((2, 1), np.float32), k, scale=1.0)
    for r in range(2):
        ref = (k[r] @ q[r, 0]).astype(np.float32)
        np.testing.assert_allclose(got[r], ref, rtol=1e-6, atol=1e-5)


def test_scores_weights_select_heads():
    """w = e_h isolates head h: the score equals head h's own dot products (mat-vec)."""
    g = np.random.default_rng(4)
    H = 6
    q = g.standard_normal((1, H, 128))
    k = g.standard_normal((1, 64, 128))
    for h in range(H):
        w = np.zeros((1, H), np.float32)
        w[0, h] = 1.0
        got = oracle.index_score(q, w, k, scale=1.0)
        np.testing.assert_allclose(got[0], (k[0] @ q[0, h]).astype(np.float32), rtol=1e-6, atol=1e-5)


def test_scores_scale_is_linear():
    g = np.random.default_rng(5)
    q = g.standard_normal((2, 4, 128))
    k = g.standard_normal((2, 40, 128))
    w = g.standard_normal((2, 4)).astype(np.float32)
    a = oracle.index_score(q, w, k, scale=1.0)
    b = oracle.index_score(q, w, k, scale=2.0)
    assert np.array_equal(b, 2 * a)  # x2 is exact in binary


def _sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("relu", [False, True])
def test_scores_hadamard_invariance(relu):
    """q_H . k_H = q H H^T k = 128 q . k for the unnormalised Sylvester H of order 128
    (its orthogonality is why dropping the rotation is a no-op on scores).  Small
    integer inputs keep every product and sum exact, so the relation holds exactly."""
    g = np.random.default_rng(6)
    H = _sylvester(128)
    q = np.zeros((2, 3, 128))
    k = np.zeros((2, 20, 128))
    for arr in (q, k):
        flat = arr.reshape(-1, 128)
        for row in flat:
            nz = g.choice(128, size=4, replace=False)
            row[nz] = g.integers(-2, 3, size=4)
    w = np.array([[1, -2, 3], [0.5, 1, -1]], np.float32)
    base = oracle.index_score(q, w, k, scale=1.0, positions=np.array([19, 10], np.int32), relu=relu)
    rot = oracle.index_score(q @ H, w, k @ H, scale=1.0, positions=np.array([19, 10], np.int32), relu=relu)
    valid = base > -1e30
    assert np.array_equal(rot[valid], 128 * base[valid])
    assert np.array_equal(rot[~valid], base[~valid])


def test_scores_fp8_keys_decode_and_scale():
    """FP8 keys: k = value(code) * scale[slot].  Codes 0x38 (1.0) and 0xB8 (-1.0), 0x7E (448)
    and scales 0.25 / 2 / 1/448 give hand-computable dot products with q = ones."""
    codes = np.zeros((1, 3, 128), np.uint8)
    codes[0, 0, :] = 0x38      # 1.0 everywhere
    codes[0, 1, :64] = 0xB8    # -1.0 in the first half
    codes[0, 2, 5] = 0x7E      # 448 in one element
    scales = np.array([[0.25, 2.0, 1.0 / 448.0]], np.float32)
    q = np.ones((1, 1, 128))
    got = oracle.index_score(q, np.ones((1, 1), np.float32), codes, k_scale=scales, scale=1.0)
    exp = np.array([[128 * 0.25, -64 * 2.0, 448 * float(np.float32(1 / 448))]], np.float32)
    assert np.array_equal(got, exp)


def test_scores_fp8_equals_decoded_f64():
    g = np.random.default_rng(7)
    codes = g.integers(0, 256, size=(2, 30, 128), dtype=np.uint16).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00  # no NaN codes
    scales = g.uniform(0.01, 2.0, size=(2, 30)).astype(np.float32)
    q = torch.from_numpy(g.standard_normal((2, 4, 128)).astype(np.float32)).to(torch.bfloat16)
    w = g.standard_normal((2, 4)).astype(np.float32)
    a = oracle.index_score(q, w, codes, k_scale=scales, scale=0.3)
    kd = oracle.decode_fp8_e4m3(codes) * scales[..., None].astype(np.float64)
    b = oracle.index_score(q, w, kd, scale=0.3)
    assert np.array_equal(a, b)


def test_scores_masked_slots_exact_and_finite():
    g = np.random.default_rng(8)
    q = g.standard_normal((3, 2, 128))
    k = g.standard_normal((3, 70, 128))
    pos = np.array([0, 33, 69], np.int32)
    s = oracle.index_score(q, np.ones((3, 2), np.float32), k, scale=1.0, positions=pos)
    mb = np.float32(oracle.mask_bound())
    for r, p in enumerate(pos):
        assert np.all(s[r, p + 1:] == mb)
        assert np.all(s[r, : p + 1] > -1e30)
    assert np.isfinite(s).all()
