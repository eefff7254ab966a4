"""GPU parity of dsa_sparse_attn_masked_dense against the oracle's masked dense attention
(OpenXLA tokamax "Supported Ops and Hardware", masked_dense_mla row), needs an MI355X.

Both attention kernels are reached (few query tokens: the list split over workgroups; 256 tokens:
one workgroup per token and head group), with ragged S_kv, lists holding -1, out-of-range and
repeated entries, sinks of either sign and none, a selection that covers the whole sequence, and
an empty one.  On lists without repeats the masked-dense form is also compared with dsa_sparse_attn.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check_attn

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


def _inputs(seed, B, S, Hq, Dqk, S_kv, K_top, masked=0.1, dup=0.1, oob=0.03, sink="normal", replace=True):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, S, Hq, Dqk)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy((g.standard_normal((B, S_kv, Dqk)) * 0.5).astype(np.float32)).to(torch.bfloat16)
    idx = np.stack([np.stack([g.choice(S_kv, size=K_top, replace=replace or K_top > S_kv) for _ in range(S)])
                    for _ in range(B)]).astype(np.int32)
    r = g.random(idx.shape)
    idx[r < masked] = -1
    idx[(r >= masked) & (r < masked + oob)] = S_kv + 7
    if dup > 0:
        d = g.random(idx.shape) < dup
        idx[d] = idx[..., :1].repeat(K_top, -1)[d]
    if sink == "normal":
        sk = torch.from_numpy(g.standard_normal(Hq).astype(np.float32))
    elif sink is None:
        sk = None
    else:
        sk = torch.full((Hq,), float(sink), dtype=torch.float32)
    return q, kv, sk, torch.from_numpy(idx)


def _case(dsa, label, q, kv, sk, idx, sm_scale, Dv):
    B, S, Hq, Dqk = q.shape
    announce("dsa_sparse_attn_masked_dense %s B=%d S=%d Hq=%d Dqk=%d Dv=%d S_kv=%d K_top=%d" % (
        label, B, S, Hq, Dqk, Dv, kv.shape[1], idx.shape[2]))
    out, lse = dsa.dsa_sparse_attn_masked_dense(_cuda(q), _cuda(kv), _cuda(sk), _cuda(idx), sm_scale=sm_scale,
                                                dv=Dv, with_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.masked_dense_attn(q, kv, sk, idx, sm_scale=sm_scale, dv=Dv)
    err, rel = check_attn(out.float().cpu().numpy(), ref)
    g_lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    np.testing.assert_allclose(g_lse[fin], ref_lse[fin], rtol=1e-4, atol=1e-4)
    return out, lse


def test_masked_dense_tiny_decode_shape(dsa):
    # the small decode configuration: 1 token, 8 heads, 192 / 128, 2048 slots, a top-64 selection
    q, kv, sk, idx = _inputs(1, 1, 1, 8, 192, 2048, 64)
    _case(dsa, "tiny", q, kv, sk, idx, 192 ** -0.5, 128)


@pytest.mark.parametrize("B,S_kv,K_top", [(2, 1000, 700), (5, 3001, 1152), (3, 64, 200)])
def test_masked_dense_mla_shape_split(dsa, B, S_kv, K_top):
    # few tokens: the split kernel over a list of S_kv entries; S_kv ragged against 32-row blocks
    q, kv, sk, idx = _inputs(10 + B, B, 1, 128, 576, S_kv, K_top)
    _case(dsa, "mla split", q, kv, sk, idx, 576 ** -0.5, 512)


def test_masked_dense_many_tokens(dsa):
    # 256 query tokens x 128 heads fill the chip: the many-token kernel (no split)
    q, kv, sk, idx = _inputs(20, 1, 256, 128, 576, 1000, 300)
    assert dsa.load_library().dsa_sparse_attn_workspace_size(1, 256, 128, 512, 1000) == 0  # many-token path
    _case(dsa, "many tokens", q, kv, sk, idx, 576 ** -0.5, 512)


@pytest.mark.parametrize("sink", [None, -30.0, 30.0])
def test_masked_dense_sinks_and_small_heads(dsa, sink):
    q, kv, sk, idx = _inputs(30, 2, 3, 16, 64, 500, 120, sink=sink)
    _case(dsa, "sink=%s" % sink, q, kv, sk, idx, 0.125, 64)


def test_masked_dense_whole_sequence_and_empty(dsa):
    B, S, Hq, Dqk, S_kv = 2, 2, 16, 64, 333
    q, kv, sk, _ = _inputs(40, B, S, Hq, Dqk, S_kv, 8)
    full = torch.from_numpy(np.tile(np.arange(S_kv, dtype=np.int32)[::-1], (B, S, 1)).copy())
    _case(dsa, "every slot", q, kv, sk, full, 0.125, 64)
    empty = torch.full((B, S, 5), -1, dtype=torch.int32)
    out, lse = _case(dsa, "nothing selected", q, kv, sk, empty, 0.125, 64)
    assert torch.count_nonzero(out).item() == 0
    np.testing.assert_allclose(lse.cpu().numpy(), sk[None, None, :].expand(B, S, Hq).numpy(), rtol=1e-6, atol=1e-6)


def test_masked_dense_agrees_with_sparse_on_lists_without_repeats(dsa):
    # distinct entries: the set form and the multiset form are the same attention
    q, kv, sk, idx = _inputs(50, 4, 1, 128, 576, 2048, 1152, masked=0.05, dup=0.0, oob=0.0, replace=False)
    announce("masked dense vs dsa_sparse_attn, B=4 S_kv=2048 K_top=1152 (distinct entries)")
    a = dsa.dsa_sparse_attn_masked_dense(_cuda(q), _cuda(kv), _cuda(sk), _cuda(idx), sm_scale=576 ** -0.5, dv=512)
    b = dsa.dsa_sparse_attn(_cuda(q), _cuda(kv), _cuda(sk), _cuda(idx), sm_scale=576 ** -0.5, dv=512)
    torch.cuda.synchronize()
    check_attn(a.float().cpu().numpy(), b.float().cpu().numpy().astype(np.float64))
