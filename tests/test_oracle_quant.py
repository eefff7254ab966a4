"""Pins for the oracle's FP8 block quantiser and key-cache write (CPU only).

The recipe is the FP8 block quantiser of the kwkr.cn article on the
DeepSeek-V4-Pro-0813-nvfp4-DSpark inference/kernel.py (FP8 block quantisation
section): blocks of 128 elements, scale = amax / 448, data in E4M3's +-448,
optional power-of-two scale, optional quantise-then-dequantise.  The oracle
is checked against hand-derived codes (tests/golden/quant_small.json),
torch's own E4M3 and bfloat16 conversions (library routines the oracle does
not call), the seeded generator's independent quantiser, and error bounds
that follow from the format.
"""
import json
import os

import numpy as np
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_small.json")


def _bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_quant_golden_blocks():
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        x = np.zeros(128, np.float32)
        for i, v in case["elements"]:
            x[i] = v
        xb = _bf16(x)
        assert np.array_equal(xb.to(torch.float32).numpy(), x), case["name"]  # values exact in bfloat16
        codes, scales = oracle.quantize_fp8_blocks(xb, round_scale=case["round_scale"])
        want = np.zeros(128, np.uint8)
        for i, c in case["codes"]:
            want[i] = c
        assert scales.shape == (1,) and scales[0] == np.float32(case["scale"]), case["name"]
        assert np.array_equal(codes, want), (case["name"], np.nonzero(codes != want))


def test_encode_roundtrips_every_finite_code():
    c = _finite_codes()
    v = oracle.decode_fp8_e4m3(c).astype(np.float32)
    assert np.array_equal(oracle.encode_fp8_e4m3(v), c)  # includes -0 -> 0x80


def test_encode_matches_torch_on_midpoints_and_neighbours():
    pos = np.sort(oracle.decode_fp8_e4m3(np.arange(0x7F, dtype=np.uint8)))  # 0 .. 448
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)                     # exact in binary32
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    g = np.random.default_rng(5)
    rand = np.concatenate([g.uniform(-448, 448, 50000), g.standard_normal(50000) * 2.0 ** g.integers(-12, 8, 50000)])
    y = np.concatenate([mids, -mids, near, -near, rand.astype(np.float32)]).astype(np.float32)
    y = np.clip(y, -448, 448)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8_e4m3(y), ref)


def test_quantizer_matches_generator_recipe():
    # the seeded generator quantises with torch's cast; the oracle searches the code table
    k = synthetic.normal(77, 0, (300, 128))
    codes, scales = oracle.quantize_fp8_blocks(k)
    g_codes, g_scales = synthetic.quantize_fp8_blocks(k)
    assert np.array_equal(codes, g_codes.numpy())
    assert np.array_equal(scales[:, 0], g_scales.numpy())


def _error_bound_ok(x, codes, s):
    """|value(code) * s - x| <= half a unit in the last place of E4M3 at y = x / s,
    plus the binary32 rounding of y."""
    v = oracle.decode_fp8_e4m3(codes)
    y = x / s
    ulp = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3), 2.0 ** -9)
    return np.all(np.abs(v - y) <= ulp / 2 + np.abs(y) * 2.0 ** -23)


def test_quantizer_error_bound_and_max_element():
    g = np.random.default_rng(9)
    for mag in (1.0, 1e-30, 1e30, 3e-38):
        x = (g.standard_normal((64, 128)) * mag).astype(np.float32)
        xb = _bf16(x)
        xf = xb.to(torch.float64).numpy()
        codes, scales = oracle.quantize_fp8_blocks(xb)
        for b in range(64):
            s = float(scales[b, 0])
            amax = np.abs(xf[b]).max()
            # one binary32 rounding of amax / 448 (absolute 2^-150 where the scale is subnormal)
            assert s > 0 and abs(s - amax / 448) <= max(amax / 448 * 2.0 ** -24, 2.0 ** -150)
            assert _error_bound_ok(xf[b], codes[b], s), (mag, b)
            i = int(np.argmax(np.abs(xf[b])))
            assert codes[b, i] & 0x7F == 0x7E  # the largest element lands on +-448


def test_power_of_two_scale():
    g = np.random.default_rng(10)
    x = (g.standard_normal((200, 128)) * np.exp(g.uniform(-20, 20, (200, 1)))).astype(np.float32)
    xb = _bf16(x)
    xf = xb.to(torch.float64).numpy()
    codes, scales = oracle.quantize_fp8_blocks(xb, round_scale=True)
    for b in range(200):
        s = float(scales[b, 0])
        m, _ = np.frexp(s)
        assert m == 0.5  # a power of two
        r = np.abs(xf[b]).max() / 448
        assert r * (1 - 2.0 ** -24) <= s and s < 2 * r * (1 + 2.0 ** -23) + 2.0 ** -149
        assert _error_bound_ok(xf[b], codes[b], s)


def test_dequantize_matches_torch_conversions():
    g = np.random.default_rng(12)
    xb = _bf16(g.standard_normal((100, 128)) * 3)
    codes, scales = oracle.quantize_fp8_blocks(xb)
    ours = oracle.dequantize_fp8_blocks(codes, scales)
    prod = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scales)
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_cache_write_placement():
    g = np.random.default_rng(13)
    T, rps, S_max = 6, 3, 4
    k = _bf16(g.standard_normal((T, 128)))
    pos = np.array([0, 3, -1, 2, 4, 1], np.int32)  # token 2 (-1) and token 4 (= S_max) are skipped
    cache = np.full((2, S_max, 128), 0xAB, np.uint8)
    sc = np.full((2, S_max), -1.0, np.float32)
    new_c, new_s = oracle.cache_write(k, pos, cache, sc, rows_per_seq=rps)
    codes, scales = oracle.quantize_fp8_blocks(k)
    placed = {(0, 0): 0, (0, 3): 1, (1, 2): 3, (1, 1): 5}
    for c in range(2):
        for p in range(S_max):
            if (c, p) in placed:
                t = placed[(c, p)]
                assert np.array_equal(new_c[c, p], codes[t]) and new_s[c, p] == scales[t, 0]
            else:
                assert np.all(new_c[c, p] == 0xAB) and new_s[c, p] == -1.0
    # bf16 cache: plain copy, and quantise-then-dequantise
    bcache = np.zeros((2, S_max, 128), np.uint16)
    kbits = k.view(torch.int16).numpy().view(np.uint16)
    plain = oracle.cache_write(k, pos, bcache, rows_per_seq=rps)
    qdq = oracle.cache_write(k, pos, bcache, rows_per_seq=rps, qdq=True)
    deq = oracle.dequantize_fp8_blocks(codes, scales)
    for (c, p), t in placed.items():
        assert np.array_equal(plain[c, p], kbits[t]) and np.array_equal(qdq[c, p], deq[t])
    assert np.all(plain[1, 0] == 0) and np.all(qdq[0, 1] == 0)

