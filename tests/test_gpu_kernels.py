"""GPU parity of each entry point against the CPU oracle on seeded inputs (needs an MI355X).

Sizes are small enough for the oracle to finish in seconds while spanning
several workgroup tiles and ragged tails; the edge matrix covers empty and
ragged rows, k around n_valid, masked / out-of-range / duplicate indices,
sinks of either sign and no sink.  Full-size workloads are in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import (check_attn, check_index_list, check_scores, check_topk_same_scores, n_valid_rows)

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


# ------------------------------------------------------------------ scores

def _score_case(dsa, w, label, relu=False):
    announce("dsa_index_score %s M=%d S_max=%d H=%d fp8=%s relu=%s" % (label, w.M, w.S_max, w.index_q.shape[1],
                                                                      w.key_fp8, relu))
    got = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                              k_scale=_cuda(w.k_scale), positions=_cuda(w.positions), valid_len=w.valid_len,
                              rows_per_seq=w.rows_per_seq, relu=relu)
    torch.cuda.synchronize()
    ref = oracle.index_score(w.index_q, w.index_w, w.k_cache, k_scale=w.k_scale, scale=w.index_scale,
                             positions=w.positions, valid_len=w.valid_len, rows_per_seq=w.rows_per_seq, relu=relu)
    nv = n_valid_rows(None if w.positions is None else w.positions.numpy(), w.valid_len, w.M, w.S_max)
    return check_scores(got.cpu().numpy(), ref, nv, oracle.mask_bound())


def test_score_tiny_decode(dsa):
    _score_case(dsa, synthetic.make_workload("tiny_decode"), "tiny_decode")


@pytest.mark.parametrize("H", [1, 4, 64, 128])
def test_score_decode_bf16_edges(dsa, H):
    S_max = 5000  # not a multiple of the 512-slot chunk
    w = synthetic.make_workload("batched_decode", M=9, H=H, S_max=S_max, pos_lo=0, topk=64)
    w.positions = torch.tensor([-1, 0, 62, 63, 64, 511, 512, S_max - 2, S_max - 1], dtype=torch.int32)
    _score_case(dsa, w, "edges H=%d" % H)


def test_score_decode_valid_len_cap(dsa):
    w = synthetic.make_workload("batched_decode", M=4, S_max=3000, pos_lo=100, topk=64)
    w.valid_len = 1234
    _score_case(dsa, w, "valid_len cap")
    w.positions = None
    _score_case(dsa, w, "valid_len only")


def test_score_decode_fp8(dsa):
    w = synthetic.make_workload("fp8_long_decode", M=3, S_max=3000, vl_lo=1000, topk=64)
    _score_case(dsa, w, "fp8 scaled")


# ReLU decode: per-head MFMA scorer (heads cannot be folded)
@pytest.mark.parametrize("H", [1, 4, 16, 17, 64])
def test_score_decode_relu_edges(dsa, H):
    S_max = 5000  # a ragged last chunk and a ragged last 16-slot tile
    w = synthetic.make_workload("batched_decode", M=9, H=H, S_max=S_max, pos_lo=0, topk=64)
    w.positions = torch.tensor([-1, 0, 14, 15, 16, 511, 512, S_max - 2, S_max - 1], dtype=torch.int32)
    _score_case(dsa, w, "relu edges H=%d" % H, relu=True)


def test_score_decode_relu_multichunk(dsa):
    # 40 rows x 40 chunks: the launch gives each workgroup a run of 4 chunks
    # (2048 slots); valid lengths end on, beside and inside those runs, and
    # the last chunk of every row is ragged
    S_max = 20000
    w = synthetic.make_workload("batched_decode", M=40, H=64, S_max=S_max, pos_lo=0, topk=64)
    g = np.random.default_rng(11)
    pos = g.integers(-1, S_max, size=40)
    pos[:10] = [-1, 0, 2046, 2047, 2048, 4095, 6143, 8191, S_max - 33, S_max - 1]
    w.positions = torch.from_numpy(pos.astype(np.int32))
    _score_case(dsa, w, "relu multi-chunk runs", relu=True)
    # fp8 keys, 16 rows x 79 chunks: runs of 3 chunks, the last run short
    w = synthetic.make_workload("fp8_long_decode", M=16, S_max=40000, vl_lo=1000, topk=64)
    _score_case(dsa, w, "relu fp8 multi-chunk runs", relu=True)


def test_score_decode_relu_fp8(dsa):
    w = synthetic.make_workload("fp8_long_decode", M=3, S_max=3000, vl_lo=1000, topk=64)
    _score_case(dsa, w, "relu fp8 scaled", relu=True)
    # negative and zero slot scales: the scale multiplies the dot before the activation
    g = np.random.default_rng(3)
    w.k_scale = torch.from_numpy((g.standard_normal((3, 3000)) * 0.01).astype(np.float32))
    w.k_scale[:, ::7] = 0.0
    _score_case(dsa, w, "relu fp8 signed scales", relu=True)


def test_score_decode_fp8_all_codes(dsa):
    """Every finite E4M3 code, one-hot queries: scores = value(code) * scale exactly decoded."""
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]          # 254 finite codes
    S_max = 256
    kc = np.zeros((1, S_max, 128), np.uint8)
    kc[0, : len(codes), 5] = codes
    kc[0, : len(codes), 77] = codes[::-1]
    w = synthetic.make_workload("fp8_long_decode", M=1, S_max=S_max, vl_lo=S_max, topk=8)
    w.k_cache = torch.from_numpy(kc)
    w.k_scale = torch.full((1, S_max), 0.5, dtype=torch.float32)
    w.positions = torch.tensor([S_max - 1], dtype=torch.int32)
    _score_case(dsa, w, "fp8 all codes")


# identity: the folded-query kernel (any H up to 128); ReLU: the per-head MFMA kernel (H <= 64)
@pytest.mark.parametrize("S,H,relu", [(300, 64, False), (300, 64, True), (77, 4, False), (130, 40, True),
                                       (513, 64, False), (300, 128, False), (33, 1, False), (31, 64, True)])
def test_score_prefill_causal(dsa, S, H, relu):
    w = synthetic.make_workload("prefill", S=S, H=H, topk=64)
    announce("dsa_index_score prefill S=%d H=%d relu=%s" % (S, H, relu))
    got = dsa.dsa_index_score(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), scale=w.index_scale,
                              positions=_cuda(w.positions), rows_per_seq=w.rows_per_seq, relu=relu)
    torch.cuda.synchronize()
    ref = oracle.index_score(w.index_q, w.index_w, w.k_cache, scale=w.index_scale, positions=w.positions,
                             rows_per_seq=w.rows_per_seq, relu=relu)
    check_scores(got.cpu().numpy(), ref, np.arange(1, S + 1), oracle.mask_bound())


def test_score_prefill_several_sequences_with_offset(dsa):
    """3 sequences of 100 query rows each; each sequence's cache has 150 slots and its queries
    start at position 20 (chunked prefill); plus a valid_len cap."""
    g = np.random.default_rng(9)
    n_seq, rps, S_max, H = 3, 100, 150, 64
    q = torch.from_numpy(g.standard_normal((n_seq * rps, H, 128)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(g.standard_normal((n_seq * rps, H)).astype(np.float32))
    k = torch.from_numpy(g.standard_normal((n_seq, S_max, 128)).astype(np.float32)).to(torch.bfloat16)
    pos = torch.from_numpy(np.tile(np.arange(20, 20 + rps), n_seq).astype(np.int32))
    for vl in (-1, 90):
        announce("dsa_index_score prefill n_seq=3 rows_per_seq=100 valid_len=%d" % vl)
        got = dsa.dsa_index_score(_cuda(q), _cuda(w), _cuda(k), scale=0.1, positions=_cuda(pos), valid_len=vl,
                                  rows_per_seq=rps)
        torch.cuda.synchronize()
        ref = oracle.index_score(q, w, k, scale=0.1, positions=pos, valid_len=vl, rows_per_seq=rps)
        check_scores(got.cpu().numpy(), ref, n_valid_rows(pos.numpy(), vl, n_seq * rps, S_max), oracle.mask_bound())


# ------------------------------------------------------------------ top-k

# paths: one workgroup per row with the row in LDS (S_max <= 8192, a
# multiple of 4); fewer than 1024 rows longer than 4096 slots: the chunked
# path (a chip-wide first-digit histogram, a chip-wide filter into per-chunk
# candidate regions, a per-row resolve) over 2048-slot chunks when 4096-slot
# chunks would give fewer than 512 workgroups, else 4096-slot chunks (here
# e.g. 8 x 65536 runs 2048-slot chunks and 8 x 300000 4096-slot ones); one
# workgroup per row re-reading the row otherwise
@pytest.mark.parametrize("S_max,k", [(100, 1), (5000, 64), (33000, 1024), (65536, 2048), (40002, 512),
                                     (70000, 2048), (3000, 2048), (300000, 2048), (8192, 2048), (8188, 333)])
def test_topk_edges(dsa, S_max, k):
    g = np.random.default_rng(S_max * 7 + k)
    nvs = sorted({0, 1, max(0, k - 1), k, k + 1, S_max // 2, S_max - 1, S_max})
    nvs = [n for n in nvs if 0 <= n <= S_max]
    M = len(nvs)
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    sc[1::2] = np.round(sc[1::2] * 4) / 4  # heavy exact ties on odd rows
    sc[:, ::97] = 1e30                      # large values, also beyond n_valid
    pos = np.array(nvs, np.int32) - 1
    announce("dsa_topk S_max=%d k=%d rows=%d" % (S_max, k, M))
    idx, tsc = dsa.dsa_topk(torch.from_numpy(sc).cuda(), k, positions=torch.from_numpy(pos).cuda(), with_scores=True)
    torch.cuda.synchronize()
    idx, tsc = idx.cpu().numpy(), tsc.cpu().numpy()
    nv = np.array(nvs)
    check_topk_same_scores(idx, sc, nv, k)
    for i in range(M):
        ok = idx[i] >= 0
        assert np.array_equal(tsc[i][ok], sc[i, idx[i][ok]])
        assert np.all(np.isneginf(tsc[i][~ok]))


@pytest.mark.parametrize("M,S_max,k", [(1100, 9001, 1024), (5, 4001, 300), (1030, 10000, 2048)])
def test_topk_row_reread_path(dsa, M, S_max, k):
    """The row path that re-reads each row per digit: 1024 or more rows longer than 8192 slots, or a row
    length that is not a multiple of 4."""
    g = np.random.default_rng(M + S_max + k)
    sc = g.standard_normal((M, S_max)).astype(np.float32)
    sc[::3] = np.round(sc[::3] * 8) / 8  # exact ties on every third row
    nv = g.integers(0, S_max + 1, M)
    nv[:4] = [0, 1, k, S_max]
    pos = (nv - 1).astype(np.int32)
    announce("dsa_topk row path M=%d S_max=%d k=%d" % (M, S_max, k))
    idx, tsc = dsa.dsa_topk(torch.from_numpy(sc).cuda(), k, positions=torch.from_numpy(pos).cuda(), with_scores=True)
    torch.cuda.synchronize()
    idx, tsc = idx.cpu().numpy(), tsc.cpu().numpy()
    check_topk_same_scores(idx, sc, nv, k)
    for i in range(0, M, 97):
        ok = idx[i] >= 0
        assert np.array_equal(tsc[i][ok], sc[i, idx[i][ok]])
        assert np.all(np.isneginf(tsc[i][~ok]))


@pytest.mark.parametrize("S_max", [4000, 20000, 65536, 300000])
def test_topk_all_equal_row(dsa, S_max):
    """Every score ties: any k of them is a valid answer (row and chunked paths).  From 20000 slots the
    tied candidates exceed the select kernel's LDS list and spill to the workspace."""
    sc = np.zeros((2, S_max), np.float32)
    announce("dsa_topk all-equal rows S_max=%d" % S_max)
    idx = dsa.dsa_topk(torch.from_numpy(sc).cuda(), 1000, valid_len=S_max - 1).cpu().numpy()
    check_topk_same_scores(idx, sc, np.array([S_max - 1, S_max - 1]), 1000)


@pytest.mark.parametrize("S_max", [50000, 70000])
def test_topk_repeated_calls_reuse_workspace(dsa, S_max):
    """Back-to-back calls agree (the chunked path clears its workspace itself)."""
    g = np.random.default_rng(5)
    sc = torch.from_numpy(g.standard_normal((5, S_max)).astype(np.float32)).cuda()
    announce("dsa_topk repeated calls S_max=%d" % S_max)
    a = dsa.dsa_topk(sc, 1024)
    b = dsa.dsa_topk(sc, 1024)
    torch.cuda.synchronize()
    assert torch.equal(a, b)  # deterministic: same columns, not only the same sets
    check_topk_same_scores(a.cpu().numpy(), sc.cpu().numpy(), np.full(5, S_max), 1024)


# ------------------------------------------------------------------ sparse attention

def _attn_inputs(seed, B, S, Hq, Dqk, Dv, S_kv, K_top, masked=0.1, dup=0.0, oob=0.0, sink="normal"):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, S, Hq, Dqk)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy((g.standard_normal((B, S_kv, Dqk)) * 0.5).astype(np.float32)).to(torch.bfloat16)
    idx = np.stack([np.stack([g.choice(S_kv, size=K_top, replace=K_top > S_kv) for _ in range(S)])
                    for _ in range(B)]).astype(np.int32)
    r = g.random(idx.shape)
    idx[r < masked] = -1
    idx[(r >= masked) & (r < masked + oob)] = S_kv + 5
    if dup > 0:
        d = g.random(idx.shape) < dup
        idx[d] = idx[..., :1].repeat(idx.shape[-1], -1)[d]
    if sink == "normal":
        sk = torch.from_numpy(g.standard_normal(Hq).astype(np.float32))
    elif sink is None:
        sk = None
    else:
        sk = torch.full((Hq,), float(sink), dtype=torch.float32)
    return q, kv, sk, torch.from_numpy(idx)


def _attn_case(dsa, label, q, kv, sk, idx, sm_scale, Dv):
    B, S, Hq, Dqk = q.shape
    announce("dsa_sparse_attn %s B=%d S=%d Hq=%d Dqk=%d Dv=%d S_kv=%d K_top=%d" % (
        label, B, S, Hq, Dqk, Dv, kv.shape[1], idx.shape[2]))
    out, lse = dsa.dsa_sparse_attn(_cuda(q), _cuda(kv), _cuda(sk), _cuda(idx), sm_scale=sm_scale, dv=Dv,
                                   with_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn(q, kv, sk, idx, sm_scale=sm_scale, dv=Dv)
    err, rel = check_attn(out.float().cpu().numpy(), ref)
    g_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    np.testing.assert_allclose(g_lse[fin], ref_lse[fin], rtol=1e-4, atol=1e-4)
    return err, rel


def test_attn_tiny_decode_shape(dsa):
    q, kv, sk, idx = _attn_inputs(1, 1, 1, 8, 192, 128, 2048, 64)
    _attn_case(dsa, "tiny", q, kv, sk, idx, 192 ** -0.5, 128)


# B = 2: fewer tokens than XCDs; B = 13: more, not a multiple of 8 (the split-combine places whole
# tokens per XCD, so the last XCDs get a partial run or none); both run 8 splits of the list
@pytest.mark.parametrize("B", [2, 13])
def test_attn_full_decode_shape_split(dsa, B):
    q, kv, sk, idx = _attn_inputs(2 + B, B, 1, 128, 576, 512, 3000, 1152, masked=0.05)
    assert dsa.load_library().dsa_sparse_attn_workspace_size(B, 1, 128, 512, 1152) > 0  # split path
    _, rel = _attn_case(dsa, "mla-shaped split", q, kv, sk, idx, 576 ** -0.5, 512)
    assert rel < 2e-2


@pytest.mark.parametrize("K_top", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("sink", [None, -30.0, 0.0, 30.0])
def test_attn_ktop_and_sink(dsa, K_top, sink):
    q, kv, sk, idx = _attn_inputs(3 + K_top, 2, 2, 16, 64, 64, 500, K_top, masked=0.2, sink=sink)
    _attn_case(dsa, "K_top=%d sink=%s" % (K_top, sink), q, kv, sk, idx, 0.125, 64)


# Value widths that end in half a 32-feature tile, head counts that are not a multiple of the
# 32 heads of a wave, and both workgroup shapes: few tokens (waves share 32 heads and split
# each block's entries; list split over workgroups) and 300 tokens (each wave owns 32 of a
# workgroup's 128 heads and every entry).
@pytest.mark.parametrize("B,S,Hq,Dqk,Dv", [(3, 1, 40, 96, 80), (2, 2, 8, 32, 16), (300, 1, 40, 96, 80),
                                           (2, 150, 128, 576, 512), (1, 300, 130, 192, 128)])
def test_attn_odd_shapes(dsa, B, S, Hq, Dqk, Dv):
    q, kv, sk, idx = _attn_inputs(11 + Hq, B, S, Hq, Dqk, Dv, 600, 300, masked=0.1)
    _, rel = _attn_case(dsa, "odd shape", q, kv, sk, idx, Dqk ** -0.5, Dv)
    assert rel < 2e-2


def test_attn_index_patterns(dsa):
    q, kv, sk, idx = _attn_inputs(4, 3, 2, 24, 128, 96, 700, 300, masked=0.1, dup=0.1, oob=0.05)
    idx[0, 0, :] = -1                 # all masked
    idx[0, 1, :100] = -1              # leading -1
    idx[1, 0, -150:] = -1             # trailing -1
    idx[2, 1, :] = 699                # one slot repeated
    _attn_case(dsa, "index patterns", q, kv, sk, idx, 0.1, 96)
    _attn_case(dsa, "index patterns no sink", q, kv, None, idx, 0.1, 96)


def test_attn_peaked_softmax(dsa):
    q, kv, sk, idx = _attn_inputs(5, 2, 1, 64, 576, 512, 2000, 512)
    q = (q.float() * 8).to(torch.bfloat16)
    _, rel = _attn_case(dsa, "peaked", q, kv, sk, idx, 576 ** -0.5, 512)
    assert rel < 2e-2


@pytest.mark.parametrize("Hq,Dqk,Dv", [(128, 576, 512), (16, 192, 128), (24, 128, 96)])
def test_attn_growing_logits(dsa, Hq, Dqk, Dv):
    """Logits that keep growing along the list: every head shares a query component c, and the
    listed rows are a_j * c / |c| + noise with a_j rising from 0 to 20, so the logit of the j-th
    listed row grows by ~90 (log2 units) over the list.  A block maximum then outgrows the running
    reference many times within each split, which the kernel handles by running the list again with
    a raised reference.  The softmax ends up concentrated on the last rows."""
    B, S_kv, K_top = 2, 2000, 1152
    g = np.random.default_rng(71)
    c = g.standard_normal(Dqk)
    c *= 3.0 * Dqk ** 0.5 / np.linalg.norm(c)
    q = c[None, None, None, :] + 0.3 * g.standard_normal((B, 1, Hq, Dqk))
    a = np.linspace(0.0, 20.0, K_top)
    rows = np.stack([g.choice(S_kv, size=K_top, replace=False) for _ in range(B)])
    kv = 0.3 * g.standard_normal((B, S_kv, Dqk))
    for b in range(B):
        kv[b, rows[b]] += a[:, None] * (c / np.linalg.norm(c))[None, :]
    idx = rows[:, None, :].astype(np.int32)
    q = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(kv.astype(np.float32)).to(torch.bfloat16)
    sk = torch.from_numpy(g.standard_normal(Hq).astype(np.float32))
    _, rel = _attn_case(dsa, "growing logits", q, kv, sk, torch.from_numpy(idx), Dqk ** -0.5, Dv)
    assert rel < 2e-2
    # the same rows listed in falling order: the first block holds the maximum, no second pass
    _, rel = _attn_case(dsa, "falling logits", q, kv, sk, torch.from_numpy(idx[..., ::-1].copy()), Dqk ** -0.5,
                        Dv)
    assert rel < 2e-2


def test_attn_growing_logits_many_tokens(dsa):
    """As test_attn_growing_logits with 300 query tokens of one sequence (the kernel for calls whose
    tokens fill the chip): every token lists the same 512 rows in rising order of a_j, so the
    reference max of every head is outgrown several times along the list."""
    S, Hq, Dqk, Dv, S_kv, K_top = 300, 32, 192, 128, 1000, 512
    g = np.random.default_rng(73)
    c = g.standard_normal(Dqk)
    c *= 3.0 * Dqk ** 0.5 / np.linalg.norm(c)
    q = c[None, None, None, :] + 0.3 * g.standard_normal((1, S, Hq, Dqk))
    a = np.linspace(0.0, 20.0, K_top)
    rows = g.choice(S_kv, size=K_top, replace=False)
    kv = 0.3 * g.standard_normal((1, S_kv, Dqk))
    kv[0, rows] += a[:, None] * (c / np.linalg.norm(c))[None, :]
    idx = np.broadcast_to(rows[None, None, :], (1, S, K_top)).astype(np.int32).copy()
    idx[0, ::7, ::5] = -1  # some masked entries on some tokens
    q = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(kv.astype(np.float32)).to(torch.bfloat16)
    sk = torch.from_numpy(g.standard_normal(Hq).astype(np.float32))
    _, rel = _attn_case(dsa, "growing logits, many tokens", q, kv, sk, torch.from_numpy(idx), Dqk ** -0.5, Dv)
    assert rel < 2e-2


# Prefill-shaped attention: many query tokens of one sequence, each with its own causal list
@pytest.mark.parametrize("S,topk,Hq,Dqk,Dv", [(200, 128, 128, 576, 512), (300, 64, 16, 192, 128),
                                              (130, 100, 24, 128, 96)])
def test_attn_prefill_causal_lists(dsa, S, topk, Hq, Dqk, Dv):
    w = synthetic.make_workload("prefill_attn", S=S, topk=topk, Hq=Hq, Dqk=Dqk, Dv=Dv)
    _, rel = _attn_case(dsa, "prefill causal lists", w.q, w.kv, w.sink, w.index_list, w.sm_scale, Dv)
    assert rel < 2e-2


# ------------------------------------------------------------------ decode step

def _decode_case(dsa, w, label, relu=False):
    announce("dsa_decode_step %s B=%d S_max=%d topk=%d window=%d Hq=%d Dqk=%d relu=%s" % (
        label, w.M, w.S_max, w.index_topk, w.window, w.q.shape[2], w.q.shape[3], relu))
    step = dsa.dsa_decode_step(_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache), k_scale=_cuda(w.k_scale),
                               positions=_cuda(w.positions), valid_len=w.valid_len, index_scale=w.index_scale,
                               index_topk=w.index_topk, window=w.window, q=_cuda(w.q), kv=_cuda(w.kv),
                               attn_sink=_cuda(w.sink), sm_scale=w.sm_scale, dv=w.dv, relu=relu)
    torch.cuda.synchronize()
    pos = None if w.positions is None else w.positions.numpy()
    nv = n_valid_rows(pos, w.valid_len, w.M, w.S_max)
    ref_sc = oracle.index_score(w.index_q, w.index_w, w.k_cache, k_scale=w.k_scale, scale=w.index_scale,
                                positions=w.positions, valid_len=w.valid_len, relu=relu)
    check_scores(step.scores.cpu().numpy(), ref_sc, nv, oracle.mask_bound())
    ref_top = oracle.topk(ref_sc, w.index_topk, positions=w.positions, valid_len=w.valid_len)
    ref_list = oracle.assemble(ref_top, s_max=w.S_max, window=w.window, positions=w.positions,
                               valid_len=w.valid_len)
    gpu_list = step.index_list.cpu().numpy()
    check_index_list(gpu_list, ref_list, ref_sc, nv, w.index_topk, w.window)
    # attention on the list the step built (validated just above): where scores tie at the k-th
    # largest, the GPU may keep another tied slot than the oracle, and then attends to other rows
    ref_out, _ = oracle.sparse_attn(w.q, w.kv, w.sink, gpu_list[:, None, :], sm_scale=w.sm_scale, dv=w.dv)
    err, rel = check_attn(step.out.float().cpu().numpy(), ref_out)
    return step, ref_sc, ref_list


def test_decode_step_tiny(dsa):
    _decode_case(dsa, synthetic.make_workload("tiny_decode"), "tiny_decode")


def test_decode_step_mla_scaled(dsa):
    w = synthetic.make_workload("full_decode_step", B=3, S_max=3000, topk=256, window=128)
    w.positions = torch.tensor([2999, 100, 1500], dtype=torch.int32)
    _decode_case(dsa, w, "scaled full step")


def test_decode_step_relu(dsa):
    """ReLU indexer (per-head scorer) through the whole step; the top-k then clears its own workspace."""
    _decode_case(dsa, synthetic.make_workload("tiny_decode"), "tiny_decode", relu=True)
    w = synthetic.make_workload("full_decode_step", B=3, S_max=9000, topk=512, window=128)
    w.positions = torch.tensor([8999, 100, 4500], dtype=torch.int32)
    _decode_case(dsa, w, "scaled full step", relu=True)


def test_decode_step_fp8_keys(dsa):
    w = synthetic.make_workload("full_decode_step", B=2, S_max=2000, topk=128, window=16, Hq=16, Dqk=192, Dv=128)
    from synthetic.gen import quantize_fp8_blocks

    codes, scales = quantize_fp8_blocks(w.k_cache.float())
    w.k_cache, w.k_scale = codes, scales
    _decode_case(dsa, w, "fp8 keys")
