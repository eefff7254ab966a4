"""Pins for the oracle's sparse attention with sink (CPU only).

Checks against hand-derived values, closed forms (one entry -> logistic
weight; q = 0 -> mean), a library softmax (no-sink case), the dense-mask
formulation of the same contract (NeMo AutoModel deepseek_v4 page,
dense_attention_topk_torch), the blockwise online-softmax algorithm the
DeepSeek-V4 kernel uses (kwkr.cn article on DeepSeek-V4-Pro inference/
kernel.py, sparse-attention section: 64-entry blocks, running max and
sum-exp rescaled by exp(old max - new max), sink added to the denominator at
the end), and the set / -1 invariances.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _rand_case(seed, B=2, S=2, Hq=4, Dqk=64, Dv=48, S_kv=300, K_top=150, frac_masked=0.1):
    g = np.random.default_rng(seed)
    q = _bf16(g.standard_normal((B, S, Hq, Dqk)))
    kv = _bf16(g.standard_normal((B, S_kv, Dqk)) * 0.5)
    sink = g.standard_normal(Hq).astype(np.float32)
    idx = np.stack([np.stack([g.permutation(S_kv)[:K_top] for _ in range(S)]) for _ in range(B)]).astype(np.int32)
    idx[g.random(idx.shape) < frac_masked] = -1
    return q, kv, sink, idx


def test_attn_golden(golden_dir):
    with open(os.path.join(golden_dir, "attn_small.json")) as f:
        c = json.load(f)["case"]
    sink = np.array([math.log(2.0), 0.0], np.float32)
    out, lse = oracle.sparse_attn(np.array(c["q"], np.float64), np.array(c["kv"], np.float64), sink,
                                  np.array(c["idx"], np.int32), sm_scale=math.log(3.0), dv=c["dv"])
    # the sink is stored in fp32: ln2 carries a 2e-8 relative rounding
    np.testing.assert_allclose(out, np.array(c["expected_out"]), rtol=1e-7)
    np.testing.assert_allclose(lse, np.array(c["expected_lse"]), rtol=1e-7)


def test_attn_single_entry_is_logistic():
    g = np.random.default_rng(21)
    q = g.standard_normal((1, 1, 3, 32))
    kv = g.standard_normal((1, 10, 32))
    sink = np.array([-1.0, 0.5, 2.0], np.float32)
    idx = np.full((1, 1, 8), -1, np.int32)
    idx[0, 0, 5] = 7
    out, lse = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.3, dv=16)
    for h in range(3):
        logit = 0.3 * float(q[0, 0, h] @ kv[0, 7])
        w = 1.0 / (1.0 + math.exp(float(sink[h]) - logit))
        np.testing.assert_allclose(out[0, 0, h], w * kv[0, 7, :16], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0, h], logit + math.log1p(math.exp(float(sink[h]) - logit)), rtol=1e-12)
    out_ns, _ = oracle.sparse_attn(q, kv, None, idx, sm_scale=0.3, dv=16)
    for h in range(3):
        assert np.array_equal(out_ns[0, 0, h], kv[0, 7, :16])  # weight exactly 1


def test_attn_zero_query_is_mean():
    g = np.random.default_rng(22)
    kv = g.standard_normal((1, 40, 16))
    idx = np.array([[[3, 9, 1, 30, -1, 22]]], np.int32)
    sink = np.array([0.7], np.float32)
    out, lse = oracle.sparse_attn(np.zeros((1, 1, 1, 16)), kv, sink, idx, sm_scale=1.0, dv=16)
    n = 5
    exp = kv[0, [3, 9, 1, 30, 22]].mean(axis=0) * n / (n + math.exp(float(sink[0])))
    np.testing.assert_allclose(out[0, 0, 0], exp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(n + math.exp(float(sink[0]))), rtol=1e-12)


def test_attn_no_sink_is_library_softmax():
    q, kv, _, idx = _rand_case(23, frac_masked=0.0)
    out, _ = oracle.sparse_attn(q, kv, None, idx, sm_scale=0.125, dv=48)
    qd, kvd = q.double().numpy(), kv.double().numpy()
    for b in range(2):
        for s in range(2):
            sel = kvd[b, idx[b, s]]
            for h in range(4):
                p = scipy.special.softmax(0.125 * sel @ qd[b, s, h])
                np.testing.assert_allclose(out[b, s, h], p @ sel[:, :48], rtol=1e-10, atol=1e-13)


def test_attn_sink_minus_inf_reduces_to_plain_softmax():
    q, kv, _, idx = _rand_case(24)
    a, la = oracle.sparse_attn(q, kv, None, idx, sm_scale=0.2, dv=48)
    b, lb = oracle.sparse_attn(q, kv, np.full(4, -np.inf, np.float32), idx, sm_scale=0.2, dv=48)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_attn_all_masked():
    q, kv, sink, idx = _rand_case(25)
    idx[:] = -1
    idx[0, 0, :10] = 300  # == S_kv: out of range, masked too
    out, lse = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.2, dv=48)
    assert np.all(out == 0.0)
    assert np.array_equal(lse, np.broadcast_to(sink.astype(np.float64), lse.shape))
    _, lse2 = oracle.sparse_attn(q, kv, None, idx, sm_scale=0.2, dv=48)
    assert np.all(np.isneginf(lse2))


def test_attn_permutation_and_minus_one_invariance():
    q, kv, sink, idx = _rand_case(26)
    a, la = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.2, dv=48)
    g = np.random.default_rng(0)
    perm = idx[..., g.permutation(idx.shape[-1])]
    b, lb = oracle.sparse_attn(q, kv, sink, perm, sm_scale=0.2, dv=48)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lb, la, rtol=1e-13)
    # inserting -1 entries anywhere keeps the valid entries in the same order: exact
    ext = np.full(idx.shape[:-1] + (idx.shape[-1] * 2,), -1, np.int32)
    ext[..., 1::2] = idx
    c, lc = oracle.sparse_attn(q, kv, sink, ext, sm_scale=0.2, dv=48)
    assert np.array_equal(c, a) and np.array_equal(lc, la)


def test_attn_duplicates_count_as_multiset():
    g = np.random.default_rng(27)
    q = g.standard_normal((1, 1, 1, 8))
    kv = g.standard_normal((1, 5, 8))
    sink = np.array([0.3], np.float32)
    out, _ = oracle.sparse_attn(q, kv, sink, np.array([[[2, 2, 4]]], np.int32), sm_scale=1.0, dv=8)
    l2, l4 = float(q[0, 0, 0] @ kv[0, 2]), float(q[0, 0, 0] @ kv[0, 4])
    e2, e4, es = 2 * math.exp(l2), math.exp(l4), math.exp(0.3 * 1.0 if False else float(sink[0]))
    exp = (e2 * kv[0, 2] + e4 * kv[0, 4]) / (e2 + e4 + es)
    np.testing.assert_allclose(out[0, 0, 0], exp, rtol=1e-12)


def test_attn_gather_equals_dense_mask_form():
    """Duplicate-free index lists: the gather form equals masked dense attention over all
    S_kv slots with the sink as an extra logit carrying a zero value row."""
    q, kv, sink, idx = _rand_case(28)
    out, lse = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.15, dv=48)
    qd, kvd = q.double().numpy(), kv.double().numpy()
    for b in range(2):
        for s in range(2):
            mask = np.zeros(300, bool)
            mask[idx[b, s][idx[b, s] >= 0]] = True
            logits = 0.15 * kvd[b] @ qd[b, s].T          # [S_kv, Hq]
            logits[~mask] = -np.inf
            full = np.concatenate([logits, sink[None, :].astype(np.float64)], axis=0)
            p = scipy.special.softmax(full, axis=0)
            vals = np.concatenate([kvd[b][:, :48], np.zeros((1, 48))], axis=0)
            np.testing.assert_allclose(out[b, s], p.T @ vals, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(lse[b, s], scipy.special.logsumexp(full, axis=0), rtol=1e-12)


def _online_blockwise(q, kv, sink, idx, sm_scale, dv, block=64):
    """The blockwise algorithm: per 64-entry block gather (masked entries -> -inf score,
    zero row), update running max and sum-exp with exp(old - new) rescaling, accumulate
    P @ V, add the sink's exp(sink - max) to the denominator after the last block."""
    B, S, Hq, _ = q.shape
    out = np.zeros((B, S, Hq, dv))
    for b in range(B):
        for s in range(S):
            m = np.full(Hq, -np.inf)
            l = np.zeros(Hq)
            acc = np.zeros((Hq, dv))
            lst = idx[b, s]
            for j0 in range(0, len(lst), block):
                blk = lst[j0:j0 + block]
                ok = (blk >= 0) & (blk < kv.shape[1])
                rows = np.where(ok[:, None], kv[b, np.clip(blk, 0, kv.shape[1] - 1)], 0.0)
                sc = sm_scale * q[b, s] @ rows.T                 # [Hq, block]
                sc[:, ~ok] = -np.inf
                m_new = np.maximum(m, sc.max(axis=1))
                alpha = np.where(np.isneginf(m_new), 1.0, np.exp(m - np.where(np.isneginf(m_new), 0, m_new)))
                p = np.where(np.isneginf(m_new)[:, None], 0.0, np.exp(sc - m_new[:, None]))
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ rows[:, :dv]
                m = m_new
            denom = l + (np.exp(sink - m) if sink is not None else 0.0)
            out[b, s] = np.where(denom[:, None] > 0, acc / np.where(denom > 0, denom, 1)[:, None], 0.0)
    return out


@pytest.mark.parametrize("with_sink", [True, False])
def test_attn_two_pass_equals_online_blockwise(with_sink):
    q, kv, sink, idx = _rand_case(29, K_top=200)
    sk = sink if with_sink else None
    out, _ = oracle.sparse_attn(q, kv, sk, idx, sm_scale=0.25, dv=48)
    ref = _online_blockwise(q.double().numpy(), kv.double().numpy(),
                            None if sk is None else sk.astype(np.float64), idx, 0.25, 48)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_attn_threads_do_not_change_results():
    q, kv, sink, idx = _rand_case(30)
    a, la = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.2, dv=48, nthreads=1)
    b, lb = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.2, dv=48, nthreads=5)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
