"""Repeated calls on the same inputs give bitwise-identical results (needs an MI355X).

Every kernel fixes its summation order and every output position (prefix
sums, not atomics, place the top-k entries), so scores, top-k rows (column
for column, ties included), attention outputs and the whole decode step are
reproducible.  Each case runs twice, with other work in between so that the
second call does not find the first one's workspace or caches untouched.
"""
import numpy as np
import pytest
import torch

import synthetic

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


def _same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape
    ab = a.contiguous().view(torch.uint8) if a.dtype != torch.bool else a
    bb = b.contiguous().view(torch.uint8) if b.dtype != torch.bool else b
    assert torch.equal(ab, bb), "%s differs between two calls" % what


def _disturb():
    """Unrelated device work between the two calls (reuses the allocator's blocks)."""
    x = torch.randn(1 << 22, device="cuda")
    (x * 3).sum().item()


@pytest.mark.parametrize("name,relu", [("batched_decode", False), ("batched_decode", True),
                                       ("fp8_long_decode", False)])
def test_decode_scores_and_topk_repeat(dsa, name, relu):
    if name == "batched_decode":
        w = synthetic.make_workload(name, M=8, S_max=40000, pos_lo=20000, topk=1024)
    else:
        w = synthetic.make_workload(name, M=3, S_max=70000, vl_lo=30000, topk=2048)
    announce("determinism: dsa_index_score + dsa_topk %s relu=%s" % (name, relu))
    args = (_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache))
    kw = dict(scale=w.index_scale, k_scale=_cuda(w.k_scale), positions=_cuda(w.positions), valid_len=w.valid_len,
              relu=relu)
    s1 = dsa.dsa_index_score(*args, **kw)
    t1, v1 = dsa.dsa_topk(s1, w.index_topk, positions=_cuda(w.positions), with_scores=True)
    _disturb()
    s2 = dsa.dsa_index_score(*args, **kw)
    t2, v2 = dsa.dsa_topk(s2, w.index_topk, positions=_cuda(w.positions), with_scores=True)
    torch.cuda.synchronize()
    _same(s1, s2, "scores")
    _same(t1, t2, "top-k row")
    _same(v1, v2, "top-k scores")


@pytest.mark.parametrize("S_max,M", [(3000, 6), (6000, 1200), (9001, 1030), (50000, 4), (300000, 8)])
def test_topk_ties_repeat(dsa, S_max, M):
    """Heavy exact ties at the boundary on every path (row in LDS, row re-read, chunked with 2048- and
    4096-slot chunks): the tie-break is the same on every call."""
    g = np.random.default_rng(S_max + M)
    sc = torch.from_numpy((np.round(g.standard_normal((M, S_max)) * 3) / 3).astype(np.float32)).cuda()
    announce("determinism: dsa_topk ties S_max=%d M=%d" % (S_max, M))
    a = dsa.dsa_topk(sc, 1000)
    _disturb()
    b = dsa.dsa_topk(sc, 1000)
    torch.cuda.synchronize()
    _same(a, b, "top-k row")


def test_prefill_scores_and_topk_repeat(dsa):
    for relu in (False, True):
        w = synthetic.make_workload("prefill", S=2048, H=64, topk=512)
        announce("determinism: prefill dsa_index_score + dsa_topk 2048 rows relu=%s" % relu)
        args = (_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache))
        kw = dict(scale=w.index_scale, positions=_cuda(w.positions), rows_per_seq=w.rows_per_seq, relu=relu)
        s1 = dsa.dsa_index_score(*args, **kw)
        t1 = dsa.dsa_topk(s1, w.index_topk, positions=_cuda(w.positions))
        _disturb()
        s2 = dsa.dsa_index_score(*args, **kw)
        t2 = dsa.dsa_topk(s2, w.index_topk, positions=_cuda(w.positions))
        torch.cuda.synchronize()
        _same(s1, s2, "prefill scores")
        _same(t1, t2, "prefill top-k row")


@pytest.mark.parametrize("B,S,Hq,Dqk,Dv,K_top", [(64, 1, 128, 576, 512, 1152),   # decode: split list + combine
                                                 (2, 1, 16, 192, 128, 300),      # decode, one split
                                                 (1, 300, 128, 576, 512, 512)])  # many tokens: wide kernel
def test_attention_repeat(dsa, B, S, Hq, Dqk, Dv, K_top):
    g = np.random.default_rng(B * S + K_top)
    S_kv = 4096
    q = torch.from_numpy(g.standard_normal((B, S, Hq, Dqk)).astype(np.float32)).to(torch.bfloat16).cuda()
    kv = torch.from_numpy((0.5 * g.standard_normal((B, S_kv, Dqk))).astype(np.float32)).to(torch.bfloat16).cuda()
    sink = torch.from_numpy(g.standard_normal(Hq).astype(np.float32)).cuda()
    idx = g.integers(0, S_kv, (B, S, K_top)).astype(np.int32)
    idx[g.random(idx.shape) < 0.05] = -1
    idx = torch.from_numpy(idx).cuda()
    announce("determinism: dsa_sparse_attn B=%d S=%d Hq=%d %d/%d K_top=%d" % (B, S, Hq, Dqk, Dv, K_top))
    o1, l1 = dsa.dsa_sparse_attn(q, kv, sink, idx, sm_scale=Dqk ** -0.5, dv=Dv, with_lse=True)
    _disturb()
    o2, l2 = dsa.dsa_sparse_attn(q, kv, sink, idx, sm_scale=Dqk ** -0.5, dv=Dv, with_lse=True)
    torch.cuda.synchronize()
    _same(o1, o2, "attention output")
    _same(l1, l2, "attention lse")


@pytest.mark.parametrize("relu", [False, True])
def test_decode_step_repeat(dsa, relu):
    """The fused step at 16 x 32768 (chunked top-k, split attention) and the tiny step (row top-k)."""
    for w in (synthetic.make_workload("full_decode_step", B=16, S_max=32768, topk=1024, window=128),
              synthetic.make_workload("tiny_decode")):
        announce("determinism: dsa_decode_step %s B=%d S_max=%d relu=%s" % (w.name, w.M, w.S_max, relu))
        step = dsa.DecodeStep(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), positions=_cuda(w.positions),
                              valid_len=w.valid_len, index_scale=w.index_scale, index_topk=w.index_topk,
                              window=w.window, q=_cuda(w.q), kv=_cuda(w.kv), attn_sink=_cuda(w.sink),
                              sm_scale=w.sm_scale, dv=w.dv, relu=relu)
        step()
        first = [t.clone() for t in (step.scores, step.index_list, step.out, step.lse)]
        _disturb()
        step()
        torch.cuda.synchronize()
        for a, b, what in zip(first, (step.scores, step.index_list, step.out, step.lse),
                              ("scores", "index list", "output", "lse")):
            _same(a, b, "decode step " + what)


@pytest.mark.parametrize("static_scratch", [False, True])
def test_decode_step_graph_replays(dsa, static_scratch):
    """A step captured in a HIP graph: every replay equals an eager step on the same inputs, with eager work and
    synchronisations between replays, and replays follow inputs rewritten in place (new positions)."""
    w = synthetic.make_workload("full_decode_step", B=16, S_max=32768, topk=1024, window=128)
    announce("graph replay: dsa_decode_step B=%d S_max=%d static_scratch=%s" % (w.M, w.S_max, static_scratch))
    ins = dict(index_q=_cuda(w.index_q), index_w=_cuda(w.index_w), k_cache=_cuda(w.k_cache),
               positions=_cuda(w.positions), q=_cuda(w.q), kv=_cuda(w.kv), attn_sink=_cuda(w.sink))
    kw = dict(valid_len=w.valid_len, index_scale=w.index_scale, index_topk=w.index_topk, window=w.window,
              sm_scale=w.sm_scale, dv=w.dv)
    eager = dsa.DecodeStep(ins["index_q"], ins["index_w"], ins["k_cache"], positions=ins["positions"],
                           q=ins["q"], kv=ins["kv"], attn_sink=ins["attn_sink"], **kw)
    graphed = dsa.DecodeStep(ins["index_q"], ins["index_w"], ins["k_cache"], positions=ins["positions"],
                             q=ins["q"], kv=ins["kv"], attn_sink=ins["attn_sink"], static_scratch=static_scratch,
                             graph=True, **kw)
    outs = lambda st: (st.scores, st.index_list, st.out, st.lse)
    g = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(4):
        if rep == 2:  # new positions, written in place into the buffer both steps read
            ins["positions"].copy_(torch.randint(1000, w.S_max, (w.M,), generator=g, dtype=torch.int32))
        eager()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs(eager)]
        _disturb()
        graphed()
        torch.cuda.synchronize()
        for a, b, what in zip(ref, outs(graphed), ("scores", "index list", "output", "lse")):
            _same(a, b, "graph replay %d %s" % (rep, what))
        _disturb()
        torch.cuda.synchronize()


def test_workspace_contents_do_not_matter(dsa):
    """Whatever the caller's workspace holds on entry (here all 0xFF bytes, then zeros), the results are the
    same: every call clears the state it accumulates into (the top-k histograms and counters) itself, and the
    attention's split partials are written before they are read."""
    g = np.random.default_rng(11)
    sc = torch.from_numpy(g.standard_normal((8, 50000)).astype(np.float32)).cuda()
    nws = dsa.topk_workspace_bytes(8, 50000, 1000)
    assert nws > 0  # the chunked path
    announce("workspace contents: dsa_topk 8 x 50000 k=1000")
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    a = dsa.dsa_topk(sc, 1000, workspace=ws).clone()
    ws.zero_()
    b = dsa.dsa_topk(sc, 1000, workspace=ws)
    torch.cuda.synchronize()
    _same(a, b, "top-k row")

    S_kv, K_top = 2048, 1152
    for B in (64, 8):  # two splits, eight splits
        q = torch.from_numpy(g.standard_normal((B, 1, 128, 576)).astype(np.float32)).to(torch.bfloat16).cuda()
        kv = torch.from_numpy((0.5 * g.standard_normal((B, S_kv, 576))).astype(np.float32)).to(torch.bfloat16).cuda()
        sink = torch.from_numpy(g.standard_normal(128).astype(np.float32)).cuda()
        idx = torch.from_numpy(g.integers(-1, S_kv, (B, 1, K_top)).astype(np.int32)).cuda()
        nws = dsa.sparse_attn_workspace_bytes(B, 1, 128, 512, K_top)
        assert nws > 0  # split lists
        announce("workspace contents: dsa_sparse_attn B=%d K_top=%d" % (B, K_top))
        ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
        o1, l1 = dsa.dsa_sparse_attn(q, kv, sink, idx, sm_scale=576 ** -0.5, dv=512, with_lse=True, workspace=ws)
        o1, l1 = o1.clone(), l1.clone()
        ws.zero_()
        o2, l2 = dsa.dsa_sparse_attn(q, kv, sink, idx, sm_scale=576 ** -0.5, dv=512, with_lse=True, workspace=ws)
        torch.cuda.synchronize()
        _same(o1, o2, "attention output")
        _same(l1, l2, "attention lse")

    w = synthetic.make_workload("full_decode_step", B=16, S_max=32768, topk=1024, window=128)
    announce("workspace contents: dsa_decode_step B=16 S_max=32768")
    step = dsa.DecodeStep(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), positions=_cuda(w.positions),
                          valid_len=w.valid_len, index_scale=w.index_scale, index_topk=w.index_topk,
                          window=w.window, q=_cuda(w.q), kv=_cuda(w.kv), attn_sink=_cuda(w.sink),
                          sm_scale=w.sm_scale, dv=w.dv)
    step._ws.fill_(0xFF)
    step()
    first = [t.clone() for t in (step.index_list, step.out, step.lse)]
    step._ws.zero_()
    step()
    torch.cuda.synchronize()
    for a, b, what in zip(first, (step.index_list, step.out, step.lse), ("index list", "output", "lse")):
        _same(a, b, "decode step " + what)
