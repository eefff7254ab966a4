"""Pins for the oracle's masked dense attention (CPU only).

OpenXLA tokamax "Supported Ops and Hardware", Attention Variants table,
masked_dense_mla row: the attention restricted to the selected subset of KV
positions through a dense mask.  Checked against a scipy softmax over every
slot with the sink as an extra logit (the dense-mask form written out with a
library routine), against the gather form (``oracle.sparse_attn``) on lists
without repeats and on de-duplicated lists, and on the set properties
(order, repeats, -1 and out-of-range entries select nothing extra).
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _case(seed, B=2, S=2, Hq=4, Dqk=64, Dv=48, S_kv=300, K_top=150, masked=0.1, dup=0.2, oob=0.05):
    g = np.random.default_rng(seed)
    q = _bf16(g.standard_normal((B, S, Hq, Dqk)))
    kv = _bf16(g.standard_normal((B, S_kv, Dqk)) * 0.5)
    sink = g.standard_normal(Hq).astype(np.float32)
    idx = g.integers(0, S_kv, size=(B, S, K_top)).astype(np.int32)  # drawn with repeats
    r = g.random(idx.shape)
    idx[r < masked] = -1
    idx[(r >= masked) & (r < masked + oob)] = S_kv + 3
    d = g.random(idx.shape) < dup
    idx[d] = idx[..., :1].repeat(K_top, -1)[d]
    return q, kv, sink, idx


def _scipy_dense(q, kv, sink, idx, sm_scale, dv):
    qd, kvd = q.double().numpy(), kv.double().numpy()
    B, S, Hq, _ = qd.shape
    S_kv = kvd.shape[1]
    out = np.zeros((B, S, Hq, dv))
    lse = np.zeros((B, S, Hq))
    for b in range(B):
        for s in range(S):
            sel = idx[b, s][(idx[b, s] >= 0) & (idx[b, s] < S_kv)]
            mask = np.zeros(S_kv, bool)
            mask[sel] = True
            logits = sm_scale * kvd[b] @ qd[b, s].T  # [S_kv, Hq]
            logits[~mask] = -np.inf
            full = np.concatenate([logits, sink[None, :].astype(np.float64)], axis=0)
            p = scipy.special.softmax(full, axis=0)
            vals = np.concatenate([kvd[b][:, :dv], np.zeros((1, dv))], axis=0)
            out[b, s] = p.T @ vals
            lse[b, s] = scipy.special.logsumexp(full, axis=0)
    return out, lse


def test_masked_dense_matches_scipy_dense_softmax():
    q, kv, sink, idx = _case(71)
    out, lse = oracle.masked_dense_attn(q, kv, sink, idx, sm_scale=0.15, dv=48)
    ref, ref_lse = _scipy_dense(q, kv, sink, idx, 0.15, 48)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_masked_dense_equals_gather_form_on_deduplicated_lists():
    q, kv, sink, idx = _case(72)
    dedup = np.full_like(idx, -1)
    for b in range(idx.shape[0]):
        for s in range(idx.shape[1]):
            u = np.unique(idx[b, s][(idx[b, s] >= 0) & (idx[b, s] < kv.shape[1])])
            dedup[b, s, :len(u)] = u
    out, lse = oracle.masked_dense_attn(q, kv, sink, idx, sm_scale=0.2, dv=48)
    g_out, g_lse = oracle.sparse_attn(q, kv, sink, dedup, sm_scale=0.2, dv=48)
    np.testing.assert_allclose(out, g_out, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse, g_lse, rtol=1e-12)
    # the gather form counts every entry: with repeats in the list the two differ
    r_out, _ = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.2, dv=48)
    assert np.abs(r_out - out).max() > 1e-3


def test_masked_dense_set_invariances():
    q, kv, sink, idx = _case(73, masked=0.0, dup=0.0, oob=0.0)
    out, lse = oracle.masked_dense_attn(q, kv, sink, idx, sm_scale=0.1, dv=48)
    g = np.random.default_rng(5)
    perm = idx[..., g.permutation(idx.shape[-1])]
    extra = np.concatenate([perm, perm[..., :20], np.full(idx.shape[:2] + (7,), -1, np.int32),
                            np.full(idx.shape[:2] + (3,), 10 ** 6, np.int32)], axis=-1)
    out2, lse2 = oracle.masked_dense_attn(q, kv, sink, extra, sm_scale=0.1, dv=48)
    np.testing.assert_array_equal(out2, out)  # same mask, same slot-order sums
    np.testing.assert_array_equal(lse2, lse)


@pytest.mark.parametrize("with_sink", [True, False])
def test_masked_dense_nothing_selected(with_sink):
    q, kv, sink, _ = _case(74)
    idx = np.full((2, 2, 9), -1, np.int32)
    idx[..., 4] = 10 ** 6
    out, lse = oracle.masked_dense_attn(q, kv, sink if with_sink else None, idx, sm_scale=0.1, dv=48)
    assert np.all(out == 0.0)
    if with_sink:
        np.testing.assert_array_equal(lse, np.broadcast_to(sink.astype(np.float64), lse.shape))
    else:
        assert np.all(np.isneginf(lse))


def test_masked_dense_every_slot_is_plain_softmax_attention():
    """All slots selected, no sink: softmax(q K^T) V over the whole sequence (numpy)."""
    g = np.random.default_rng(75)
    q = g.standard_normal((1, 1, 3, 16))
    kv = g.standard_normal((1, 40, 16))
    idx = np.arange(40, dtype=np.int32)[None, None, ::-1].copy()
    out, lse = oracle.masked_dense_attn(q, kv, None, idx, sm_scale=0.25, dv=16)
    logits = 0.25 * q[0, 0] @ kv[0].T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out[0, 0], p @ kv[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(logits, axis=1), rtol=1e-13)
