"""dsa_decode_step_static (scratch in a library-owned device array, no allocation) against dsa_decode_step.

Two calls in a row on the same GPU, the second with a smaller input, so the
second runs over what the first left in the shared scratch array.  Both
entry points run the same kernels; the comparison is to the parity bar:
scores bit-exact, index lists equal as sets (top-k part) and exactly (window
part), attention outputs within 2e-2 absolute (the list order inside a row
may differ between calls, which changes only the summation order).
"""
import ctypes

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


def _steps(dsa, w, relu=False):
    kw = dict(k_scale=_cuda(w.k_scale), positions=_cuda(w.positions), valid_len=w.valid_len,
              index_scale=w.index_scale, index_topk=w.index_topk, window=w.window, q=_cuda(w.q), kv=_cuda(w.kv),
              attn_sink=_cuda(w.sink), sm_scale=w.sm_scale, dv=w.dv, relu=relu)
    args = (_cuda(w.index_q), _cuda(w.index_w), _cuda(w.k_cache))
    ref = dsa.DecodeStep(*args, **kw)
    got = dsa.DecodeStep(*args, static_scratch=True, **kw)
    return ref, got


def _compare(ref, got, topk):
    sr, sg = ref.scores.cpu().numpy(), got.scores.cpu().numpy()
    assert np.array_equal(sr.view(np.uint32), sg.view(np.uint32)), "scores differ"
    lr, lg = ref.index_list.cpu().numpy(), got.index_list.cpu().numpy()
    assert np.array_equal(np.sort(lr[:, :topk], axis=1), np.sort(lg[:, :topk], axis=1)), "top-k sets differ"
    assert np.array_equal(lr[:, topk:], lg[:, topk:]), "window entries differ"
    orf, og = ref.out.float().cpu().numpy(), got.out.float().cpu().numpy()
    assert np.isfinite(og).all()
    err = float(np.abs(orf - og).max())
    assert err <= 2e-2, "attention outputs differ by %g" % err
    lr_, lg_ = ref.lse.cpu().numpy(), got.lse.cpu().numpy()
    assert float(np.abs(lr_ - lg_).max()) <= 1e-3
    return err


def test_static_scratch_two_calls_second_smaller(dsa):
    # first call: split attention (partials in scratch) and the chunked top-k (header and candidates in scratch)
    w1 = synthetic.make_workload("full_decode_step", B=16, S_max=24576, topk=1024, window=128)
    ref1, got1 = _steps(dsa, w1)
    need1 = dsa.load_library().dsa_decode_step_workspace_size(ctypes.byref(got1._args))
    assert 0 < need1 <= dsa.DSA_STATIC_SCRATCH_BYTES
    announce("dsa_decode_step_static B=16 S_max=24576 topk=1024 window=128 scratch=%d bytes" % need1)
    ref1()
    got1()
    torch.cuda.synchronize()
    e1 = _compare(ref1, got1, 1024)

    # second call, smaller, over the first call's leftovers; ReLU indexer (the other scorer)
    w2 = synthetic.make_workload("full_decode_step", B=3, S_max=5000, topk=256, window=64, seed=7)
    w2.positions = torch.tensor([4999, 40, 2500], dtype=torch.int32)
    ref2, got2 = _steps(dsa, w2, relu=True)
    announce("dsa_decode_step_static B=3 S_max=5000 topk=256 window=64 relu")
    ref2()
    got2()
    torch.cuda.synchronize()
    e2 = _compare(ref2, got2, 256)

    # the first shape again: stale contents of the smaller call must not leak into it
    got1()
    torch.cuda.synchronize()
    e3 = _compare(ref1, got1, 1024)
    print("[no-alloc] max attention differences %.3g %.3g %.3g" % (e1, e2, e3), flush=True)


def test_static_scratch_rejects_oversize(dsa):
    w = synthetic.make_workload("full_decode_step", B=2, S_max=4096, topk=64, window=8, Hq=16, Dqk=192, Dv=128)
    _, got = _steps(dsa, w)
    a = got._args
    saved = (a.B, a.S_max, a.scores, a.index_list)
    # workspace of 1024 sequences x 65536 slots kept in scratch: far above the array
    a.B, a.S_max, a.scores, a.index_list = 1024, 65536, None, None
    lib = dsa.load_library()
    assert lib.dsa_decode_step_workspace_size(ctypes.byref(a)) > dsa.DSA_STATIC_SCRATCH_BYTES
    assert lib.dsa_decode_step_static(ctypes.byref(a), None) == 5  # DSA_ERR_WORKSPACE, nothing enqueued
    a.B, a.S_max, a.scores, a.index_list = saved
    got()
    torch.cuda.synchronize()
