"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Where the oracle cannot redo the whole workload in seconds, it computes
sampled rows / sequences one by one (always including the first and last
rows and rows around tile boundaries) and the rest is checked through
properties that hold at any size (finite scores, exact mask bound, valid
top-k sets).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import (check_attn, check_index_list, check_scores, check_topk_own_scores, n_valid_rows)

pytestmark = pytest.mark.gpu


def announce(msg):
    print("\n[gpu case] " + msg, flush=True)


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_amd as m

    m.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return m


def _cuda(t):
    return None if t is None else t.contiguous().cuda()


def _decode_indexer(dsa, w, rows):
    """Score + top-k of a decode indexer workload on the GPU; oracle on `rows`."""
    pos = None if w.positions is None else w.positions.numpy()
    nv = n_valid_rows(pos, w.valid_len, w.M, w.S_max)
    scores = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                                 k_scale=_cuda(w.k_scale), positions=_cuda(w.positions), valid_len=w.valid_len)
    idx = dsa.dsa_topk(scores, w.index_topk, positions=_cuda(w.positions), valid_len=w.valid_len)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    mb = np.float32(oracle.mask_bound())
    assert np.isfinite(sc).all()
    for r in range(w.M):  # properties on every row
        assert np.all(sc[r, nv[r]:] == mb)
    rows = np.asarray(rows)
    sub_pos = None if w.positions is None else w.positions[rows]
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache[rows],
                             k_scale=None if w.k_scale is None else w.k_scale[rows], scale=w.index_scale,
                             positions=sub_pos, valid_len=w.valid_len)
    check_scores(sc[rows], ref, nv[rows], oracle.mask_bound())
    check_topk_own_scores(idx.cpu().numpy()[rows], ref, nv[rows], w.index_topk)


def test_fullsize_batched_decode(dsa):
    w = synthetic.make_workload("batched_decode")
    announce("batched_decode full: 16 x 32768 slots, 64 heads, top-1024 (all rows)")
    _decode_indexer(dsa, w, range(w.M))


def test_fullsize_batched_decode_relu(dsa):
    w = synthetic.make_workload("batched_decode")
    announce("batched_decode full, ReLU indexer: 16 x 32768 slots, 64 heads (sampled rows)")
    pos = w.positions.numpy()
    nv = n_valid_rows(pos, w.valid_len, w.M, w.S_max)
    scores = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                                 positions=_cuda(w.positions), relu=True)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    assert np.isfinite(sc).all()
    for r in range(w.M):
        assert np.all(sc[r, nv[r]:] == np.float32(oracle.mask_bound()))
    rows = np.array([0, 5, 15])
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache[rows], scale=w.index_scale,
                             positions=w.positions[rows], relu=True)
    check_scores(sc[rows], ref, nv[rows], oracle.mask_bound())


def test_fullsize_fp8_long_decode(dsa):
    w = synthetic.make_workload("fp8_long_decode")
    announce("fp8_long_decode full: 4 x 131072 fp8 slots, 64 heads, top-2048 (all rows)")
    _decode_indexer(dsa, w, range(w.M))


def _prefill_sample_rows(S, seed=73):
    """Rows of the 8192-row prefill checked against the oracle.

    The folded scorer gives a workgroup 16-row tile a and its partner tile n - 1 - a; inside a
    tile, row i sits in lane group (i % 8) / 4 of accumulator register i / 8 (hi) or i / 8 + 2 (lo);
    key tiles are 32 slots wide, so the causal limit of row r crosses a key-tile edge at r = 32 m - 1.
    The sample holds the first and last two tiles, the middle pair, every row position inside a
    tile for pairs drawn across the sequence (with the partner row taken at another position),
    and rows on both sides of 16- and 32-row edges."""
    nt = S // 16
    g = np.random.default_rng(seed)
    rows = set(range(0, 32)) | set(range(S - 32, S)) | set(range(16 * (nt // 2 - 1), 16 * (nt // 2 + 1)))
    tiles = g.choice(np.arange(2, nt // 2 - 1), size=64, replace=False)
    for j, a in enumerate(tiles):
        rows.add(16 * int(a) + j % 16)                  # every in-tile position, over the drawn tiles
        rows.add(16 * (nt - 1 - int(a)) + (j + 5) % 16)  # the partner tile, at another position
    for m in g.choice(np.arange(1, S // 32), size=24, replace=False):
        rows.update((32 * int(m) - 1, 32 * int(m), 32 * int(m) + 16))
    return np.array(sorted(r for r in rows if 0 <= r < S))


def test_fullsize_prefill(dsa):
    w = synthetic.make_workload("prefill")
    S = w.S_max
    announce("prefill full: 8192 queries x 8192 keys causal, 64 heads, top-2048 (>= 256 sampled rows)")
    scores = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                                 positions=_cuda(w.positions), rows_per_seq=w.rows_per_seq)
    idx = dsa.dsa_topk(scores, w.index_topk, positions=_cuda(w.positions))
    torch.cuda.synchronize()
    rows = _prefill_sample_rows(S)
    assert len(rows) >= 256
    sc = scores[torch.from_numpy(rows).cuda()].cpu().numpy()
    # all 8192 rows share one cache: the oracle rows map to it with rows_per_seq = len(rows)
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache, scale=w.index_scale,
                             positions=w.positions[rows], rows_per_seq=len(rows))
    check_scores(sc, ref, rows + 1, oracle.mask_bound())
    check_topk_own_scores(idx.cpu().numpy()[rows], ref, rows + 1, w.index_topk)
    full = scores.cpu().numpy()
    assert np.isfinite(full).all()
    tri = np.triu(np.ones((64, 64), bool), 1)  # spot-check the mask bound above the diagonal
    assert np.all(full[:64, :64][tri] == np.float32(oracle.mask_bound()))


def test_fullsize_prefill_relu(dsa):
    """The per-head (ReLU) prefill scorer at 8192 x 8192 on sampled rows: its workgroups take 4
    consecutive rows, its stages 128 keys in 32-key sub-tiles, and a row's scores leave a stage
    behind the next stage's key copy; the sample holds the first and last rows, every in-group
    row position, and rows whose causal limit falls on either side of a stage or sub-tile edge."""
    w = synthetic.make_workload("prefill")
    S = w.S_max
    g = np.random.default_rng(91)
    rows = set(range(0, 8)) | set(range(S - 8, S))
    for j, grp in enumerate(g.choice(np.arange(2, S // 4 - 2), size=32, replace=False)):
        rows.add(4 * int(grp) + j % 4)
    for m in g.choice(np.arange(1, S // 128), size=12, replace=False):
        rows.update((128 * int(m) - 1, 128 * int(m), 128 * int(m) + 31, 128 * int(m) + 32))
    rows = np.array(sorted(rows))
    announce("prefill full, ReLU per-head scorer: 8192 queries x 8192 keys causal, 64 heads (%d sampled rows)"
             % len(rows))
    scores = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                                 positions=_cuda(w.positions), rows_per_seq=w.rows_per_seq, relu=True)
    torch.cuda.synchronize()
    sc = scores[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache, scale=w.index_scale,
                             positions=w.positions[rows], rows_per_seq=len(rows), relu=True)
    check_scores(sc, ref, rows + 1, oracle.mask_bound())
    full = scores.cpu().numpy()
    assert np.isfinite(full).all()


def test_fullsize_decode_step(dsa):
    w = synthetic.make_workload("full_decode_step")
    announce("full_decode_step full: 64 x 65536 slots, top-1024 + window 128, 128 heads, 576/512 (sampled)")
    step = dsa.dsa_decode_step(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), positions=_cuda(w.positions),
                               valid_len=w.valid_len, index_scale=w.index_scale, index_topk=w.index_topk,
                               window=w.window, q=_cuda(w.q), kv=_cuda(w.kv), attn_sink=_cuda(w.sink),
                               sm_scale=w.sm_scale, dv=w.dv)
    torch.cuda.synchronize()
    rows = np.array([0, 17, 42, 63])
    nv = n_valid_rows(w.positions.numpy(), w.valid_len, w.M, w.S_max)
    ref_sc = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache[rows], scale=w.index_scale,
                                positions=w.positions[rows])
    check_scores(step.scores.cpu().numpy()[rows], ref_sc, nv[rows], oracle.mask_bound())
    ref_top = oracle.topk(ref_sc, w.index_topk, positions=w.positions[rows])
    ref_list = oracle.assemble(ref_top, s_max=w.S_max, window=w.window, positions=w.positions[rows])
    gpu_list = step.index_list.cpu().numpy()[rows]
    check_index_list(gpu_list, ref_list, ref_sc, nv[rows], w.index_topk, w.window)
    # attention on the list the step built (validated above; tied slots may differ from the oracle's)
    ref_out, _ = oracle.sparse_attn(w.q[rows], w.kv[rows], w.sink, gpu_list[:, None, :], sm_scale=w.sm_scale,
                                    dv=w.dv)
    check_attn(step.out.float().cpu().numpy()[rows], ref_out)
    out = step.out.float().cpu().numpy()
    assert np.isfinite(out).all()
    lst = step.index_list.cpu().numpy()
    for b in range(w.M):  # every sequence: a valid, duplicate-free list with the exact window
        live = lst[b][lst[b] >= 0]
        assert len(np.unique(live)) == len(live) and live.max() < nv[b]
        assert np.array_equal(lst[b, w.index_topk:], np.arange(nv[b] - w.window, nv[b]))


def test_fullsize_fp8_cache_write():
    """The long-context fp8 cache (4 x 131072 slots) quantised on the GPU from bf16 keys, in one call;
    the oracle requantises 4096 sampled slots (first, last and random) and they must match bit for bit."""
    import sparse_attention_amd as dsa

    n_seq, S_max = 4, 131072
    keys = synthetic.normal(41, 0, (n_seq * S_max, 128))
    pos = np.tile(np.arange(S_max, dtype=np.int32), n_seq)
    announce("dsa_cache_write fp8 full: %d x %d slots from bf16 keys (sampled check)" % (n_seq, S_max))
    kc = torch.empty((n_seq, S_max, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty((n_seq, S_max), dtype=torch.float32, device="cuda")
    dsa.dsa_cache_write(keys.cuda(), torch.from_numpy(pos).cuda(), kc, k_scale=ks, rows_per_seq=S_max)
    torch.cuda.synchronize()
    g = np.random.default_rng(42)
    rows = np.unique(np.concatenate([[0, S_max - 1, n_seq * S_max - 1], g.integers(0, n_seq * S_max, 4093)]))
    want_c, want_s = oracle.quantize_fp8_blocks(keys[torch.from_numpy(rows)])
    got_c = kc.view(-1, 128)[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_s = ks.view(-1)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got_c, want_c)
    assert np.array_equal(got_s, want_s[:, 0])


def test_fullsize_prefill_attn(dsa):
    """Prefill-shaped sparse attention at full size (8192 queries, causal top-2048 lists, 128 heads,
    576 / 512), in bench.py's launch configuration; the oracle recomputes sampled query tokens."""
    w = synthetic.make_workload("prefill_attn")
    S = w.q.shape[1]
    announce("prefill_attn full: %d queries x top-%d, 128 heads, 576/512 (sampled tokens)" % (S, w.index_topk))
    out = dsa.dsa_sparse_attn(_cuda(w.q), _cuda(w.kv), _cuda(w.sink), _cuda(w.index_list), sm_scale=w.sm_scale,
                              dv=w.dv)
    torch.cuda.synchronize()
    g = np.random.default_rng(61)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 2047, 2048, 4095, S - 1], g.integers(0, S, 8)]))
    sl = torch.from_numpy(rows)
    ref, _ = oracle.sparse_attn(w.q[:, sl], w.kv, w.sink, w.index_list[:, sl], sm_scale=w.sm_scale, dv=w.dv)
    check_attn(out[:, sl.cuda()].float().cpu().numpy(), ref)
    assert bool(torch.isfinite(out.float()).all())
