"""The parity comparators catch the mistakes they are meant to catch (CPU only).

Each case plants a plausible kernel mistake in an oracle result and checks
that the comparator in tests/parity.py rejects it, while the correctly
rounded oracle result passes:
  * attention that silently drops one 32-entry block of a 1152-entry list
    (the full decode step's list length): elementwise errors stay far below
    2e-2 because the outputs are small, the per-row relative L2 gate fails;
  * an empty list that returns anything but zeros;
  * top-k rows and index lists padded with a value other than -1.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check_attn, check_index_list, check_topk_own_scores


def _bf16_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _decode_attn_case(seed=3, B=2, Hq=8, Dqk=576, Dv=512, S_kv=4096, K_top=1152):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, 1, Hq, Dqk)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy((0.5 * g.standard_normal((B, S_kv, Dqk))).astype(np.float32)).to(torch.bfloat16)
    sink = g.standard_normal(Hq).astype(np.float32)
    idx = np.stack([g.permutation(S_kv)[:K_top] for _ in range(B)]).astype(np.int32)[:, None, :]
    return q, kv, sink, idx


def test_rel_l2_gate_catches_a_dropped_block():
    q, kv, sink, idx = _decode_attn_case()
    sm = 576 ** -0.5
    ref, _ = oracle.sparse_attn(q, kv, sink, idx, sm_scale=sm, dv=512)
    good = _bf16_round(ref)
    err, rel = check_attn(good, ref)
    assert rel < 5e-3
    dropped = idx.copy()
    dropped[:, :, 320:352] = -1  # one 32-entry block lost
    bad, _ = oracle.sparse_attn(q, kv, sink, dropped, sm_scale=sm, dv=512)
    bad = _bf16_round(bad)
    assert np.abs(bad - ref).max() < 2e-2  # the elementwise bound alone would pass it
    with pytest.raises(AssertionError, match="rel-L2"):
        check_attn(bad, ref)


def test_rel_l2_gate_empty_rows_must_be_zero():
    q, kv, sink, idx = _decode_attn_case(B=1, Hq=4, Dqk=64, Dv=32, S_kv=100, K_top=16)
    idx[:] = -1
    ref, _ = oracle.sparse_attn(q, kv, sink, idx, sm_scale=0.125, dv=32)
    assert np.all(ref == 0.0)
    check_attn(np.zeros_like(ref), ref)
    wrong = np.zeros_like(ref)
    wrong[0, 0, 1, 3] = 1e-3
    with pytest.raises(AssertionError, match="no attendable entry"):
        check_attn(wrong, ref)


def test_padding_must_be_minus_one():
    g = np.random.default_rng(5)
    nv, k = np.array([5, 40]), 8
    sc = g.standard_normal((2, 40))
    top = oracle.topk(sc, k, valid_len=-1, positions=np.array([4, 39], np.int32))
    check_topk_own_scores(top, sc, nv, k)
    bad = top.copy()
    bad[0, bad[0] == -1] = -2
    with pytest.raises(AssertionError):
        check_topk_own_scores(bad, sc, nv, k)

    window = 4
    lst = oracle.assemble(top, s_max=40, window=window, positions=np.array([4, 39], np.int32))
    check_index_list(lst, lst, sc, nv, k, window)
    bad = lst.copy()
    row0 = bad[0, :k]
    row0[row0 == -1] = -7
    with pytest.raises(AssertionError):
        check_index_list(bad, lst, sc, nv, k, window)
