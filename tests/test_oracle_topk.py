"""Pins for the oracle's top-k selection and window assembly (CPU only).

Top-k is checked against hand-derived rows, against numpy's own sort (a
library routine), and against the defining properties of the selected set.
Assembly is checked against hand-derived lists.
"""
import json
import os

import numpy as np
import pytest

import oracle


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "topk_assemble_small.json")) as f:
        return json.load(f)


def test_topk_golden(golden_dir):
    for case in _golden(golden_dir)["topk"]:
        sc = np.array([case["scores"]], np.float32)
        got = oracle.topk(sc, case["k"], valid_len=case["n_valid"])
        assert got[0].tolist() == case["expected_sorted"], case


def test_assemble_golden(golden_dir):
    for case in _golden(golden_dir)["assemble"]:
        t = np.array([case["topk"]], np.int32)
        got = oracle.assemble(t, s_max=case["n_valid"], window=case["window"], valid_len=case["n_valid"])
        assert got[0].tolist() == case["expected"], case


@pytest.mark.parametrize("S_max,k", [(100, 1), (100, 10), (1000, 64), (5000, 1024), (3000, 2048)])
def test_topk_matches_numpy_sort(S_max, k):
    g = np.random.default_rng(S_max + k)
    M = 4
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    pos = g.integers(0, S_max, size=M).astype(np.int32)
    got, got_sc = oracle.topk(sc, k, positions=pos, with_scores=True)
    for r in range(M):
        nv = int(pos[r]) + 1
        order = np.argsort(-sc[r, :nv], kind="stable")[:k]
        n = min(k, nv)
        assert set(got[r, :n].tolist()) == set(order.tolist())
        assert np.all(got[r, n:] == -1)
        assert np.array_equal(got_sc[r, :n], sc[r, got[r, :n]])
        assert np.all(np.isneginf(got_sc[r, n:]))


def test_topk_set_properties_random():
    g = np.random.default_rng(11)
    for trial in range(30):
        S_max = int(g.integers(1, 400))
        k = int(g.integers(1, 300))
        sc = np.round(g.standard_normal((1, S_max)) * 3).astype(np.float32)  # many exact ties
        nv = int(g.integers(0, S_max + 1))
        got = oracle.topk(sc, k, valid_len=nv)[0]
        n = min(k, nv)
        chosen = got[:n]
        assert np.all(got[n:] == -1)
        assert len(set(chosen.tolist())) == n and np.all((chosen >= 0) & (chosen < nv))
        if 0 < n < nv:
            rest = np.setdiff1d(np.arange(nv), chosen)
            assert sc[0, chosen].min() >= sc[0, rest].max()


def test_topk_ignores_slots_beyond_n_valid():
    sc = np.array([[0.0, 1.0, 2.0, 1e30, 1e30]], np.float32)
    got = oracle.topk(sc, 2, positions=np.array([2], np.int32))
    assert set(got[0].tolist()) == {1, 2}


def test_topk_k_at_least_n_valid_returns_all_valid():
    sc = np.random.default_rng(12).standard_normal((2, 50)).astype(np.float32)
    got = oracle.topk(sc, 64, positions=np.array([9, 49], np.int32))
    assert set(got[0, :10].tolist()) == set(range(10)) and np.all(got[0, 10:] == -1)
    assert set(got[1, :50].tolist()) == set(range(50)) and np.all(got[1, 50:] == -1)


def test_assemble_window_is_union_without_duplicates():
    g = np.random.default_rng(13)
    B, S_max, k, W = 6, 500, 40, 16
    pos = g.integers(0, S_max, size=B).astype(np.int32)
    sc = g.standard_normal((B, S_max)).astype(np.float32)
    t = oracle.topk(sc, k, positions=pos)
    a = oracle.assemble(t, s_max=S_max, window=W, positions=pos)
    for b in range(B):
        nv = int(pos[b]) + 1
        live = a[b][a[b] >= 0]
        assert len(set(live.tolist())) == len(live)
        expect = set(t[b][t[b] >= 0].tolist()) | set(range(max(0, nv - W), nv))
        assert set(live.tolist()) == expect
