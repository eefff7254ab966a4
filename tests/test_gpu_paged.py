"""GPU parity of the paged entry points (needs an MI355X).

Pools are built by the seeded generator's page scatter (random page order,
spare pages filled with unrelated data).  The oracle reads the pool back
through its own unpaging; the paged GPU result must match the oracle to the
usual tolerances and, because the kernels do the same arithmetic on the
same rows, the contiguous GPU result bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import check_attn, check_index_list, check_scores, n_valid_rows

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


def _paged(x, P, n_seq, n_slots, seed, spare=5):
    """(pool, table, n_pages) for a contiguous [n_seq, n_slots, ...] CPU tensor."""
    max_pages = -(-n_slots // P)
    n_pages = n_seq * max_pages + spare
    table = synthetic.page_table(seed, 11, n_seq, max_pages, n_pages)
    shape = (n_pages * P,) + tuple(x.shape[2:])
    if x.dtype == torch.uint8:
        fill = torch.from_numpy(np.random.default_rng(seed).integers(0, 126, size=shape, dtype=np.uint8))
    else:
        fill = synthetic.normal(seed, 12, shape, dtype=x.dtype)
    return synthetic.scatter_pages(x, table, P, n_pages, fill), table, n_pages


@pytest.mark.parametrize("fp8,relu,P", [(False, False, 64), (False, False, 256), (True, False, 128),
                                         (False, True, 64), (True, True, 512)])
def test_paged_scores(dsa, fp8, relu, P):
    if fp8:
        w = synthetic.make_workload("fp8_long_decode", M=5, S_max=3000, vl_lo=900, topk=64)
    else:
        w = synthetic.make_workload("batched_decode", M=5, H=64, S_max=3000, pos_lo=0, topk=64)
        w.positions = torch.tensor([-1, 63, 64, 1500, 2999], dtype=torch.int32)
    announce("dsa_index_score_paged fp8=%s relu=%s page=%d M=%d S_max=%d" % (fp8, relu, P, w.M, w.S_max))
    pool, table, n_pages = _paged(w.k_cache, P, w.M, w.S_max, seed=P + fp8)
    spool = None
    if fp8:
        spool, _, _ = _paged(w.k_scale, P, w.M, w.S_max, seed=P + fp8)
    paging = dsa.Paging(_cuda(table), P, n_pages)
    got = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(pool), scale=w.index_scale,
                              k_scale=_cuda(spool), positions=_cuda(w.positions), valid_len=w.valid_len, relu=relu,
                              paging=paging, s_max=w.S_max)
    flat = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                               k_scale=_cuda(w.k_scale), positions=_cuda(w.positions), valid_len=w.valid_len,
                               relu=relu)
    torch.cuda.synchronize()
    keys = oracle.unpage(pool, table, P, w.S_max)
    ks = oracle.unpage(spool, table, P, w.S_max) if fp8 else None
    ref = oracle.index_score(w.index_q, w.index_w, keys, k_scale=ks, scale=w.index_scale, positions=w.positions,
                             valid_len=w.valid_len, relu=relu)
    nv = n_valid_rows(None if w.positions is None else w.positions.numpy(), w.valid_len, w.M, w.S_max)
    check_scores(got.cpu().numpy(), ref, nv, oracle.mask_bound())
    assert torch.equal(got, flat)


@pytest.mark.parametrize("P", [64, 1024])
def test_paged_attn(dsa, P):
    B, S, Hq, Dqk, Dv, S_kv, K_top = 3, 2, 128, 576, 512, 3000, 700
    g = np.random.default_rng(P)
    q = synthetic.normal(70 + P, 0, (B, S, Hq, Dqk))
    kv = synthetic.normal(71 + P, 0, (B, S_kv, Dqk), sigma=0.5)
    sink = synthetic.normal(72 + P, 0, (Hq,), dtype=torch.float32)
    idx = g.integers(0, S_kv, size=(B, S, K_top)).astype(np.int32)
    idx[g.random((B, S, K_top)) < 0.1] = -1
    idx[0, 0, :5] = [S_kv, S_kv + 100, -7, 0, S_kv - 1]     # out of range, masked, both ends
    idx = torch.from_numpy(idx)
    announce("dsa_sparse_attn_paged page=%d B=%d S=%d K_top=%d" % (P, B, S, K_top))
    pool, table, n_pages = _paged(kv, P, B, S_kv, seed=P)
    paging = dsa.Paging(_cuda(table), P, n_pages)
    out, lse = dsa.dsa_sparse_attn(_cuda(q), _cuda(pool), _cuda(sink), _cuda(idx), sm_scale=Dqk ** -0.5, dv=Dv,
                                   with_lse=True, paging=paging, s_kv=S_kv)
    flat, flat_lse = dsa.dsa_sparse_attn(_cuda(q), _cuda(kv), _cuda(sink), _cuda(idx), sm_scale=Dqk ** -0.5, dv=Dv,
                                         with_lse=True)
    torch.cuda.synchronize()
    kv_back = oracle.unpage(pool, table, P, S_kv)
    ref, ref_lse = oracle.sparse_attn(q, kv_back, sink, idx, sm_scale=Dqk ** -0.5, dv=Dv)
    check_attn(out.float().cpu().numpy(), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)
    assert torch.equal(out, flat) and torch.equal(lse, flat_lse)


def test_paged_attn_pool_beyond_4gib(dsa):
    """The sequences' pages sit at the far end of a 4.8 GB KV pool (rows past 2^32 bytes, beyond what
    one 32-bit buffer offset reaches)."""
    B, S_kv, Hq, Dqk, Dv, K_top, P = 2, 4096, 64, 576, 512, 512, 64
    max_pages = S_kv // P
    n_pages = (1 << 22) // P  # 2^22 rows x 1152 B = 4.8 GB
    announce("dsa_sparse_attn_paged pool of %d rows (%.1f GB), pages at its end" % (n_pages * P,
                                                                                   n_pages * P * Dqk * 2 / 1e9))
    q = synthetic.normal(80, 0, (B, 1, Hq, Dqk))
    kv = synthetic.normal(81, 0, (B, S_kv, Dqk), sigma=0.5)
    sink = synthetic.normal(82, 0, (Hq,), dtype=torch.float32)
    g = np.random.default_rng(83)
    idx = torch.from_numpy(g.integers(0, S_kv, size=(B, 1, K_top)).astype(np.int32))
    # pages n_pages - 1, n_pages - 2, ... (reversed), all beyond the 4 GiB mark
    table = torch.arange(n_pages - 1, n_pages - 1 - B * max_pages, -1, dtype=torch.int32).view(B, max_pages)
    assert int(table.min()) * P * Dqk * 2 > (1 << 32)
    pool = torch.zeros((n_pages * P, Dqk), dtype=torch.bfloat16, device="cuda")
    pool.view(n_pages, P, Dqk)[table.flatten().long().cuda()] = kv.cuda().view(B * max_pages, P, Dqk)
    paging = dsa.Paging(_cuda(table), P, n_pages)
    out = dsa.dsa_sparse_attn(_cuda(q), pool, _cuda(sink), _cuda(idx), sm_scale=Dqk ** -0.5, dv=Dv, paging=paging,
                              s_kv=S_kv)
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attn(q, kv, sink, idx, sm_scale=Dqk ** -0.5, dv=Dv)
    check_attn(out.float().cpu().numpy(), ref)


@pytest.mark.parametrize("relu", [False, True])
def test_paged_decode_step(dsa, relu):
    w = synthetic.make_workload("full_decode_step", B=3, S_max=9000, topk=512, window=128, Hq=64,
                                position=None)
    w.positions = torch.tensor([8999, 4000, 200], dtype=torch.int32)
    P = 128
    announce("dsa_decode_step paged page=%d B=3 S_max=9000 relu=%s" % (P, relu))
    kpool, table, n_pages = _paged(w.k_cache, P, w.M, w.S_max, seed=90)
    kvpool, _, _ = _paged(w.kv, P, w.M, w.S_max, seed=90)
    paging = dsa.Paging(_cuda(table), P, n_pages)
    common = dict(positions=_cuda(w.positions), valid_len=w.valid_len, index_scale=w.index_scale,
                  index_topk=w.index_topk, window=w.window, attn_sink=_cuda(w.sink), sm_scale=w.sm_scale, dv=w.dv,
                  relu=relu)
    step = dsa.DecodeStep(_cuda(w.index_q), _cuda(w.index_w), _cuda(kpool), q=_cuda(w.q), kv=_cuda(kvpool),
                          paging=paging, s_max=w.S_max, **common)
    step()
    flat = dsa.DecodeStep(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), q=_cuda(w.q), kv=_cuda(w.kv),
                          **common)
    flat()
    torch.cuda.synchronize()
    assert torch.equal(step.scores, flat.scores)
    keys = oracle.unpage(kpool, table, P, w.S_max)
    kv_back = oracle.unpage(kvpool, table, P, w.S_max)
    nv = n_valid_rows(w.positions.numpy(), w.valid_len, w.M, w.S_max)
    ref_sc = oracle.index_score(w.index_q, w.index_w, keys, scale=w.index_scale, positions=w.positions, relu=relu)
    check_scores(step.scores.cpu().numpy(), ref_sc, nv, oracle.mask_bound())
    lst = step.index_list.cpu().numpy()
    ref_top = oracle.topk(ref_sc, w.index_topk, positions=w.positions, valid_len=w.valid_len)
    ref_list = oracle.assemble(ref_top, s_max=w.S_max, window=w.window, positions=w.positions, valid_len=w.valid_len)
    check_index_list(lst, ref_list, ref_sc, nv, w.index_topk, w.window)
    # attention on the step's own list (ties may pick a different valid subset than the oracle)
    ref, _ = oracle.sparse_attn(w.q, kv_back, w.sink, torch.from_numpy(lst).view(w.M, 1, -1), sm_scale=w.sm_scale,
                                dv=w.dv)
    check_attn(step.out.float().cpu().numpy(), ref)
    # the top-k is an unordered set whose order may change from run to run: same sets, and outputs
    # equal up to the summation order
    assert torch.equal(step.index_list.sort(dim=1).values, flat.index_list.sort(dim=1).values)
    check_attn(step.out.float().cpu().numpy(), flat.out.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("fp8", [False, True])
def test_paged_cache_write_then_score(dsa, fp8):
    """New keys written into a paged cache (fp8: quantised), then scored through the same table: pool bytes
    equal the oracle's cache write read back through its unpaging, and the scores match the oracle."""
    M, S_max, P = 4, 2000, 64
    w = synthetic.make_workload("batched_decode", M=M, H=64, S_max=S_max, pos_lo=0, topk=64)
    w.positions = torch.tensor([5, 1999, 64, 1000], dtype=torch.int32)
    announce("dsa_cache_write_paged fp8=%s page=%d then dsa_index_score_paged" % (fp8, P))
    keys = synthetic.normal(95, 0, (M * S_max, 128))          # every slot's key, written in one call
    pos_all = np.tile(np.arange(S_max, dtype=np.int32), M)
    max_pages = -(-S_max // P)
    n_pages = M * max_pages + 3
    table = synthetic.page_table(96, 11, M, max_pages, n_pages)
    paging = dsa.Paging(_cuda(table), P, n_pages)
    if fp8:
        pool = torch.zeros((n_pages * P, 128), dtype=torch.uint8, device="cuda")
        spool = torch.zeros((n_pages * P,), dtype=torch.float32, device="cuda")
    else:
        pool = torch.zeros((n_pages * P, 128), dtype=torch.bfloat16, device="cuda")
        spool = None
    dsa.dsa_cache_write(keys.cuda(), torch.from_numpy(pos_all).cuda(), pool, k_scale=spool, rows_per_seq=S_max,
                        paging=paging, s_max=S_max)
    got = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), pool, scale=w.index_scale, k_scale=spool,
                              positions=_cuda(w.positions), paging=paging, s_max=S_max)
    torch.cuda.synchronize()
    if fp8:
        c0 = np.zeros((M, S_max, 128), np.uint8)
        s0 = np.zeros((M, S_max), np.float32)
        want_c, want_s = oracle.cache_write(keys, pos_all, c0, s0, rows_per_seq=S_max)
        assert np.array_equal(oracle.unpage(pool, table, P, S_max), want_c)
        assert np.array_equal(oracle.unpage(spool, table, P, S_max), want_s)
        ref = oracle.index_score(w.index_q, w.index_w, want_c, k_scale=want_s, scale=w.index_scale,
                                 positions=w.positions)
    else:
        want = oracle.cache_write(keys, pos_all, np.zeros((M, S_max, 128), np.uint16), rows_per_seq=S_max)
        assert np.array_equal(oracle.unpage(pool, table, P, S_max), want)
        ref = oracle.index_score(w.index_q, w.index_w, want, scale=w.index_scale, positions=w.positions)
    nv = n_valid_rows(w.positions.numpy(), -1, M, S_max)
    check_scores(got.cpu().numpy(), ref, nv, oracle.mask_bound())
