"""Comparators between the HIP path and the CPU oracle (shared by tests, smoke and bench).

Tolerances:
  * scores: |gpu - oracle| <= 1e-3 * max(|oracle|, rms_r), rms_r = RMS of the
    oracle's attendable scores in the row (pure relative error is ill-posed
    where a score cancels to ~0); masked slots must equal the mask bound
    bit-exactly; nothing may be NaN or inf.
  * top-k: an unordered set of distinct attendable slots of the right size;
    when both sides rank the same scores the sets must be equal except among
    exactly tied scores at the k-th boundary; when the GPU ranked its own
    scores, a slot may differ from the oracle's set only if its oracle score
    lies within the score tolerance of the k-th largest.
  * attention: |gpu_bf16 - oracle| <= 2e-2 elementwise, and per (b, s, h)
    the relative L2 error ||gpu - oracle|| / ||oracle|| <= 1e-2 (a row whose
    oracle output is exactly zero, i.e. no attendable entry, must be exactly
    zero).  The elementwise bound alone would pass a kernel that dropped a
    whole block of a long list, whose outputs are small (~1e-2); the relative
    bound would not.  The measured error of correct kernels is ~3e-3 (bf16
    P and output rounding).
  * -1 padding: every entry of a top-k row or index list is either -1 or an
    attendable slot, with exactly as many -1 entries as the oracle's.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 1e-3
ATTN_ATOL = 2e-2
ATTN_REL_L2 = 1e-2


def n_valid_rows(positions, valid_len, M, S_max):
    if positions is None:
        n = np.full(M, S_max, np.int64)
    else:
        n = np.asarray(positions, np.int64) + 1
    if valid_len >= 0:
        n = np.minimum(n, valid_len)
    return np.clip(n, 0, S_max)


def check_scores(gpu: np.ndarray, ref: np.ndarray, n_valid, mask_bound: float, rows=None):
    """gpu, ref: [R, S_max] fp32 (rows `rows` of the full problem, or all)."""
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), "non-finite GPU score"
    mb = np.float32(mask_bound)
    worst = 0.0
    for i in range(gpu.shape[0]):
        nv = int(n_valid[i])
        assert np.all(gpu[i, nv:].view(np.uint32) == mb.view(np.uint32)), "row %d: masked slots differ" % i
        if nv == 0:
            continue
        o = ref[i, :nv].astype(np.float64)
        g = gpu[i, :nv].astype(np.float64)
        rms = np.sqrt(np.mean(o * o))
        tol = SCORE_RTOL * np.maximum(np.abs(o), rms)
        err = np.abs(g - o)
        bad = err > tol
        assert not bad.any(), "row %d: %d scores out of tolerance, worst slot %d gpu %r oracle %r" % (
            i, bad.sum(), int(np.argmax(err - tol)), g[np.argmax(err - tol)], o[np.argmax(err - tol)])
        worst = max(worst, float((err / np.maximum(np.maximum(np.abs(o), rms), 1e-30)).max()))
    return worst


def check_topk_same_scores(gpu_idx: np.ndarray, scores: np.ndarray, n_valid, k: int):
    """GPU top-k ranked the very scores the oracle ranks: sets equal up to exact ties."""
    for i in range(gpu_idx.shape[0]):
        nv = int(n_valid[i])
        n = min(k, nv)
        row = gpu_idx[i]
        live = row[row >= 0]
        assert len(live) == n, "row %d: %d entries, expected %d" % (i, len(live), n)
        assert np.sum(row == -1) == k - n
        assert len(np.unique(live)) == n, "row %d: duplicate index" % i
        assert np.all((live >= 0) & (live < nv)), "row %d: index outside attendable range" % i
        if n == nv:
            assert set(live.tolist()) == set(range(nv)), "row %d: expected every attendable slot" % i
            continue
        sc = scores[i, :nv]
        kth = np.partition(sc, nv - n)[nv - n]  # k-th largest value
        chosen = np.zeros(nv, bool)
        chosen[live] = True
        assert np.all(sc[chosen] >= kth), "row %d: selected a score below the k-th largest" % i
        assert np.all(sc[~chosen] <= kth), "row %d: left out a score above the k-th largest" % i
        # strictly-above-threshold slots must all be present
        assert np.all(chosen[sc > kth]), "row %d: missing a slot above the threshold" % i


def check_topk_own_scores(gpu_idx: np.ndarray, ref_scores: np.ndarray, n_valid, k: int):
    """GPU ranked its own scores: differences from the oracle's set only inside the tie band."""
    for i in range(gpu_idx.shape[0]):
        nv = int(n_valid[i])
        n = min(k, nv)
        row = gpu_idx[i]
        live = row[row >= 0]
        assert len(live) == n and len(np.unique(live)) == n
        assert np.sum(row == -1) == k - n, "row %d: padding is not exactly -1" % i
        assert np.all((live >= 0) & (live < nv))
        if n == nv:
            assert set(live.tolist()) == set(range(nv))
            continue
        o = ref_scores[i, :nv].astype(np.float64)
        vk = np.partition(o, nv - n)[nv - n]
        rms = np.sqrt(np.mean(o * o))
        tau = SCORE_RTOL * max(abs(vk), rms)
        chosen = np.zeros(nv, bool)
        chosen[live] = True
        assert np.all(o[chosen] >= vk - tau), "row %d: selected slot far below the k-th largest" % i
        assert np.all(o[~chosen] <= vk + tau), "row %d: missed slot far above the k-th largest" % i


def check_attn(gpu_out: np.ndarray, ref_out: np.ndarray, atol: float = ATTN_ATOL, rel_l2: float = ATTN_REL_L2):
    """Returns (max abs error, max relative L2 error over the (b, s, h) rows)."""
    g = np.asarray(gpu_out, np.float64)
    o = np.asarray(ref_out, np.float64)
    assert g.shape == o.shape
    assert np.isfinite(g).all()
    err = np.abs(g - o)
    assert err.max() <= atol, "attention max abs error %g > %g" % (err.max(), atol)
    num = np.sqrt((err ** 2).sum(axis=-1))
    nrm = np.sqrt((o ** 2).sum(axis=-1))
    zero = nrm == 0.0
    assert np.all(num[zero] == 0.0), "attention: %d rows with no attendable entry are not zero" % int(
        (num[zero] != 0).sum())
    rel = np.where(zero, 0.0, num / np.where(zero, 1.0, nrm))
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape) if rel.size else ()
    assert rel.size == 0 or rel.max() <= rel_l2, "attention rel-L2 error %g > %g at %s" % (rel.max(), rel_l2, worst)
    return float(err.max()), float(rel.max()) if rel.size else 0.0


def check_index_list(gpu_list: np.ndarray, ref_list: np.ndarray, ref_scores: np.ndarray, n_valid, k: int,
                     window: int):
    """Decode-step index list [B, k + window]: the window part must match exactly; the live
    entries must be distinct, the top-k part must avoid the window, and the live set may differ
    from the oracle's only by slots whose oracle scores lie in the tie band of the k-th largest."""
    assert gpu_list.shape == ref_list.shape
    assert np.array_equal(gpu_list[:, k:], ref_list[:, k:]), "window part differs"
    for b in range(gpu_list.shape[0]):
        nv = int(n_valid[b])
        wstart = nv - window
        top = gpu_list[b, :k]
        assert np.all((top == -1) | ((top >= 0) & (top < wstart))), "row %d: top-k entry inside the window" % b
        assert np.sum(top == -1) == np.sum(ref_list[b, :k] == -1), "row %d: -1 padding count differs" % b
        live = gpu_list[b][gpu_list[b] >= 0]
        assert len(np.unique(live)) == len(live), "row %d: duplicate index" % b
        G, R = set(live.tolist()), set(ref_list[b][ref_list[b] >= 0].tolist())
        if G != R:
            o = ref_scores[b, :nv].astype(np.float64)
            vk = np.sort(o)[::-1][min(k, nv) - 1]
            tau = SCORE_RTOL * max(abs(vk), float(np.sqrt(np.mean(o * o))))
            assert all(o[s] >= vk - tau for s in G - R), "row %d: extra slot outside the tie band" % b
            assert all(o[s] <= vk + tau for s in R - G), "row %d: missing slot outside the tie band" % b
            assert len(G) == len(R)
