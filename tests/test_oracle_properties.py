"""Property fuzzing of the oracle over shapes, n_valid, k and -1 patterns (CPU only).

Hypothesis draws small shapes and the edge structure the kernels must handle
(empty rows, k above n_valid, positions beyond the cache, windows wider than
the attendable range, masked, out-of-range and duplicate list entries, sinks
of either sign or none), and each case is checked against a formulation
written here independently of the oracle's C code:
  * scores: a numpy float64 evaluation of the score definition (per-head dot,
    optional ReLU, weighted head sum, scale) and the exact mask bound past
    n_valid (DeepSeek-V3.2 Sparse Indexer Kernel API Reference, Returns and
    Notes);
  * top-k: the set of the k largest attendable scores from a full numpy sort
    (lower slot first among equals, the oracle's tie rule), -1 padding;
  * index assembly: top-k entries inside the window dropped to -1, the
    window's positions appended (kwkr.cn article on DeepSeek-V4 inference,
    sparse-attention section);
  * attention: a dense softmax over the listed logits with the sink in the
    denominator (NeMo AutoModel deepseek_v4 page, sparse_attention_torch),
    and invariance to permuting the list.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _n_valid(positions, valid_len, M, S_max):
    n = np.full(M, S_max, np.int64) if positions is None else np.asarray(positions, np.int64) + 1
    if valid_len >= 0:
        n = np.minimum(n, valid_len)
    return np.clip(n, 0, S_max)


@st.composite
def score_case(draw):
    M = draw(st.integers(1, 5))
    H = draw(st.integers(1, 6))
    S_max = draw(st.integers(1, 90))
    use_pos = draw(st.booleans())
    positions = np.array([draw(st.integers(-3, S_max + 5)) for _ in range(M)], np.int32) if use_pos else None
    valid_len = draw(st.sampled_from([-1, 0, 1, S_max // 2, S_max, S_max + 7]))
    relu = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return M, H, S_max, positions, valid_len, relu, seed


@SETTINGS
@given(score_case())
def test_index_score_matches_numpy(case):
    M, H, S_max, positions, valid_len, relu, seed = case
    g = np.random.default_rng(seed)
    q = _bf16(g.standard_normal((M, H, 128)))
    w = g.standard_normal((M, H)).astype(np.float32)
    k = _bf16(g.standard_normal((M, S_max, 128)))
    got = oracle.index_score(q, w, k, scale=0.125, positions=positions, valid_len=valid_len, relu=relu)
    dots = np.einsum("mhd,msd->mhs", q.double().numpy(), k.double().numpy())
    if relu:
        dots = np.maximum(dots, 0.0)
    want = 0.125 * np.einsum("mh,mhs->ms", w.astype(np.float64), dots)
    nv = _n_valid(positions, valid_len, M, S_max)
    mb = np.float32(oracle.mask_bound())
    for r in range(M):
        assert np.all(got[r, nv[r]:].view(np.uint32) == mb.view(np.uint32))
        np.testing.assert_allclose(got[r, :nv[r]], want[r, :nv[r]], rtol=1e-6, atol=1e-5)


@st.composite
def topk_case(draw):
    M = draw(st.integers(1, 6))
    S_max = draw(st.integers(1, 120))
    k = draw(st.integers(1, 140))
    use_pos = draw(st.booleans())
    positions = np.array([draw(st.integers(-2, S_max + 3)) for _ in range(M)], np.int32) if use_pos else None
    valid_len = draw(st.sampled_from([-1, 0, 3, S_max]))
    ties = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return M, S_max, k, positions, valid_len, ties, seed


@SETTINGS
@given(topk_case())
def test_topk_is_the_k_largest_of_a_full_sort(case):
    M, S_max, k, positions, valid_len, ties, seed = case
    g = np.random.default_rng(seed)
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    if ties:
        sc = np.round(sc * 2) / 2
    got = oracle.topk(sc, k, positions=positions, valid_len=valid_len)
    nv = _n_valid(positions, valid_len, M, S_max)
    assert got.shape == (M, k)
    for r in range(M):
        n = int(min(k, nv[r]))
        order = sorted(range(int(nv[r])), key=lambda s: (-float(sc[r, s]), s))  # lower slot first among equals
        assert set(got[r, :n].tolist()) == set(order[:n])
        assert np.all(got[r, n:] == -1)


@SETTINGS
@given(topk_case(), st.integers(0, 50))
def test_assemble_window_union(case, window):
    M, S_max, k, positions, valid_len, _, seed = case
    g = np.random.default_rng(seed)
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    top = oracle.topk(sc, k, positions=positions, valid_len=valid_len)
    lst = oracle.assemble(top, s_max=S_max, window=window, positions=positions, valid_len=valid_len)
    nv = _n_valid(positions, valid_len, M, S_max)
    for r in range(M):
        ws = int(nv[r]) - window
        want_top = np.where((top[r] >= 0) & (top[r] < ws), top[r], -1)
        assert np.array_equal(lst[r, :k], want_top)
        want_win = np.array([p if p >= 0 else -1 for p in range(ws, ws + window)], np.int64)
        assert np.array_equal(lst[r, k:], want_win)
        live = lst[r][lst[r] >= 0]
        assert len(np.unique(live)) == len(live)  # a set union: no slot twice


@st.composite
def attn_case(draw):
    B = draw(st.integers(1, 2))
    S = draw(st.integers(1, 3))
    Hq = draw(st.integers(1, 5))
    Dqk = 32 * draw(st.integers(1, 4))
    Dv = 16 * draw(st.integers(1, Dqk // 16))
    S_kv = draw(st.integers(1, 60))
    K_top = draw(st.integers(1, 70))
    sink = draw(st.sampled_from(["none", "normal", "large", "very negative"]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return B, S, Hq, Dqk, Dv, S_kv, K_top, sink, seed


@SETTINGS
@given(attn_case())
def test_attention_matches_dense_softmax(case):
    B, S, Hq, Dqk, Dv, S_kv, K_top, sink_kind, seed = case
    g = np.random.default_rng(seed)
    q = _bf16(g.standard_normal((B, S, Hq, Dqk)))
    kv = _bf16(0.5 * g.standard_normal((B, S_kv, Dqk)))
    sink = None if sink_kind == "none" else {
        "normal": g.standard_normal(Hq), "large": 30 + g.standard_normal(Hq),
        "very negative": -40 + g.standard_normal(Hq)}[sink_kind].astype(np.float32)
    # masked (-1 or below), out-of-range and duplicate entries
    idx = g.integers(-3, S_kv + 3, (B, S, K_top)).astype(np.int32)
    sm = Dqk ** -0.5
    out, lse = oracle.sparse_attn(q, kv, sink, idx, sm_scale=sm, dv=Dv)
    qd, kvd = q.double().numpy(), kv.double().numpy()
    for b in range(B):
        for s in range(S):
            live = [t for t in idx[b, s] if 0 <= t < S_kv]
            for h in range(Hq):
                if not live:
                    assert np.all(out[b, s, h] == 0.0)
                    continue
                lg = sm * (kvd[b, live] @ qd[b, s, h])
                parts = np.concatenate([lg, [] if sink is None else [float(sink[h])]])
                m = parts.max()
                den = np.exp(parts - m).sum()
                want = (np.exp(lg - m) @ kvd[b, live, :Dv]) / den
                np.testing.assert_allclose(out[b, s, h], want, rtol=1e-9, atol=1e-12)
                np.testing.assert_allclose(lse[b, s, h], m + np.log(den), rtol=1e-12, atol=1e-12)
    perm = np.stack([np.stack([g.permutation(idx[b, s]) for s in range(S)]) for b in range(B)])
    out_p, _ = oracle.sparse_attn(q, kv, sink, perm, sm_scale=sm, dv=Dv)
    np.testing.assert_allclose(out_p, out, rtol=1e-12, atol=1e-14)
