"""Seeded random shapes through every entry point, against the oracle (needs an MI355X).

Each case draws its shape and edge structure from a fixed master seed:
row counts and lengths across the row, LDS-row and chunked top-k paths, k
below and above n_valid, positions before and beyond the cache, exact ties,
attention head counts and feature widths off the tuned shapes (predicated
kernel instances), lists with masked, out-of-range and duplicate entries,
sinks of either sign or none, token counts on both attention kernels, and
whole decode steps with windows, ReLU and fp8 keys.  The comparators are the
parity gates of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import check_attn, check_index_list, check_scores, check_topk_same_scores, n_valid_rows

pytestmark = pytest.mark.gpu

MASTER = 0xF0225


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


def _rng(kind, i):
    return np.random.default_rng([MASTER, kind, i])


@pytest.mark.parametrize("i", range(20))
def test_fuzz_topk(dsa, i):
    g = _rng(1, i)
    M = int(g.integers(1, 41))
    S_max = int(np.exp(g.uniform(0, np.log(70000))))
    S_max = max(S_max, 1)
    k = int(g.integers(1, 2049))
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    if g.random() < 0.5:
        sc = np.round(sc * 3) / 3  # exact ties
    pos = g.integers(-3, S_max + 10, M).astype(np.int32) if g.random() < 0.7 else None
    valid_len = int(g.integers(0, S_max + 2)) if g.random() < 0.3 else -1
    announce("fuzz dsa_topk #%d M=%d S_max=%d k=%d pos=%s valid_len=%d" % (i, M, S_max, k, pos is not None, valid_len))
    idx, tsc = dsa.dsa_topk(torch.from_numpy(sc).cuda(), k, positions=_cuda(None if pos is None else
                                                                            torch.from_numpy(pos)),
                            valid_len=valid_len, with_scores=True)
    torch.cuda.synchronize()
    idx, tsc = idx.cpu().numpy(), tsc.cpu().numpy()
    nv = n_valid_rows(pos, valid_len, M, S_max)
    check_topk_same_scores(idx, sc, nv, k)
    for r in range(M):
        ok = idx[r] >= 0
        assert np.array_equal(tsc[r][ok], sc[r, idx[r][ok]])
        assert np.all(np.isneginf(tsc[r][~ok]))


def _attn_case(g, many_tokens=False):
    if many_tokens:
        B, S = 1, int(g.integers(256, 300))
        Hq = int(g.integers(1, 131))
        Dqk = 32 * int(g.integers(1, 5))
        K_top = int(g.integers(1, 129))
    else:
        B, S = int(g.integers(1, 4)), int(g.integers(1, 5))
        Hq = int(g.integers(1, 201))
        Dqk = 32 * int(g.integers(1, 19))
        K_top = int(g.integers(1, 601))
    Dv = 16 * int(g.integers(1, min(Dqk, 512) // 16 + 1))
    S_kv = int(g.integers(1, 3001))
    q = torch.from_numpy(g.standard_normal((B, S, Hq, Dqk)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy((0.5 * g.standard_normal((B, S_kv, Dqk))).astype(np.float32)).to(torch.bfloat16)
    kind = g.integers(0, 3)
    sink = None if kind == 0 else (g.standard_normal(Hq) * (1 if kind == 1 else 8)).astype(np.float32)
    idx = g.integers(0, S_kv, (B, S, K_top)).astype(np.int32)
    r = g.random(idx.shape)
    idx[r < g.uniform(0, 0.3)] = -1
    idx[(r > 0.97)] = S_kv + 5  # out of range: masked
    if K_top > 1 and g.random() < 0.5:
        idx[..., 1] = idx[..., 0]  # duplicates count as a multiset
    if g.random() < 0.15:
        idx[0, 0, :] = -1  # a fully masked row
    return q, kv, sink, idx, Dv


@pytest.mark.parametrize("i", range(24))
def test_fuzz_sparse_attn(dsa, i):
    g = _rng(2, i)
    q, kv, sink, idx, Dv = _attn_case(g, many_tokens=(i % 6 == 5))
    B, S, Hq, Dqk = q.shape
    sm = float(Dqk) ** -0.5
    announce("fuzz dsa_sparse_attn #%d B=%d S=%d Hq=%d Dqk=%d Dv=%d S_kv=%d K_top=%d sink=%s" % (
        i, B, S, Hq, Dqk, Dv, kv.shape[1], idx.shape[2], sink is not None))
    out, lse = dsa.dsa_sparse_attn(_cuda(q), _cuda(kv), _cuda(None if sink is None else torch.from_numpy(sink)),
                                   _cuda(torch.from_numpy(idx)), sm_scale=sm, dv=Dv, with_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn(q, kv, sink, idx, sm_scale=sm, dv=Dv)
    check_attn(out.float().cpu().numpy(), ref)
    got_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.abs(got_lse[fin] - ref_lse[fin]).max(initial=0.0) <= 1e-3 * (1 + np.abs(ref_lse[fin]).max(initial=0.0))


@pytest.mark.parametrize("i", range(10))
def test_fuzz_decode_step(dsa, i):
    g = _rng(3, i)
    B = int(g.integers(1, 6))
    S_max = int(g.integers(64, 9001))
    H = int(g.integers(1, 65))
    topk = int(g.integers(1, 1025))
    window = int(g.integers(0, 201))
    Hq = int(g.integers(1, 151))
    Dqk = 32 * int(g.integers(1, 19))
    Dv = 16 * int(g.integers(1, min(Dqk, 512) // 16 + 1))
    relu = bool(g.random() < 0.4)
    fp8 = bool(g.random() < 0.3)
    w = synthetic.make_workload("full_decode_step", seed=int(g.integers(0, 2 ** 31)), B=B, H=H, S_max=S_max,
                                topk=topk, window=window, Hq=Hq, Dqk=Dqk, Dv=Dv)
    w.positions = torch.from_numpy(g.integers(-2, S_max + 50, B).astype(np.int32))
    w.valid_len = int(g.integers(0, S_max + 1)) if g.random() < 0.25 else -1
    if fp8:
        from synthetic.gen import quantize_fp8_blocks

        w.k_cache, w.k_scale = quantize_fp8_blocks(w.k_cache.float())
    announce("fuzz dsa_decode_step #%d B=%d S_max=%d H=%d topk=%d window=%d Hq=%d Dqk=%d Dv=%d relu=%s fp8=%s" % (
        i, B, S_max, H, topk, window, Hq, Dqk, Dv, relu, fp8))
    step = dsa.dsa_decode_step(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), k_scale=_cuda(w.k_scale),
                               positions=_cuda(w.positions), valid_len=w.valid_len, index_scale=w.index_scale,
                               index_topk=topk, window=window, q=_cuda(w.q), kv=_cuda(w.kv),
                               attn_sink=_cuda(w.sink), sm_scale=w.sm_scale, dv=Dv, relu=relu)
    torch.cuda.synchronize()
    nv = n_valid_rows(w.positions.numpy(), w.valid_len, B, S_max)
    ref_sc = oracle.index_score(w.index_q, w.index_w, w.k_cache, k_scale=w.k_scale, scale=w.index_scale,
                                positions=w.positions, valid_len=w.valid_len, relu=relu)
    check_scores(step.scores.cpu().numpy(), ref_sc, nv, oracle.mask_bound())
    ref_top = oracle.topk(ref_sc, topk, positions=w.positions, valid_len=w.valid_len)
    ref_list = oracle.assemble(ref_top, s_max=S_max, window=window, positions=w.positions, valid_len=w.valid_len)
    gpu_list = step.index_list.cpu().numpy()
    check_index_list(gpu_list, ref_list, ref_sc, nv, topk, window)
    ref_out, _ = oracle.sparse_attn(w.q, w.kv, w.sink, gpu_list[:, None, :], sm_scale=w.sm_scale, dv=Dv)
    check_attn(step.out.float().cpu().numpy(), ref_out)
