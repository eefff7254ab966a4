"""GPU parity of dsa_cache_write (key-cache write with FP8 block quantisation)
against the CPU oracle, bit for bit (needs an MI355X).

Codes are integers decided by binary32 arithmetic, so the bar is exact
equality of every cache byte and every scale, including slots the call must
leave alone.
"""
import numpy as np
import pytest
import torch

import oracle
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


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def _run_fp8(dsa, k_new, pos, n_seq, S_max, rows_per_seq=1, round_scale=False, seed=0):
    """Write k_new into a cache pre-filled with noise on the GPU and in the oracle; compare."""
    g = np.random.default_rng(seed)
    cache0 = g.integers(0, 256, size=(n_seq, S_max, 128), dtype=np.uint8)
    scale0 = g.standard_normal((n_seq, S_max)).astype(np.float32)
    kc = torch.from_numpy(cache0).cuda()
    ks = torch.from_numpy(scale0).cuda()
    dsa.dsa_cache_write(k_new.cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(), kc, k_scale=ks,
                        rows_per_seq=rows_per_seq, round_scale=round_scale)
    torch.cuda.synchronize()
    want_c, want_s = oracle.cache_write(k_new, pos, cache0, scale0, rows_per_seq=rows_per_seq,
                                        round_scale=round_scale)
    got_c, got_s = kc.cpu().numpy(), ks.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, "code mismatches at %s (got %s want %s)" % (
        bad[:5].tolist(), got_c[tuple(bad[:5].T)], want_c[tuple(bad[:5].T)])
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))


def _sweep_blocks(lead: float):
    """Every finite bfloat16 value with |v| <= 448, 127 per block after a lead element."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    v = _from_bits(b).to(torch.float32).numpy()
    b = b[np.abs(v) <= 448]
    n = -(-b.size // 127)
    blocks = np.zeros((n, 128), np.uint16)
    blocks[:, 1:].reshape(-1)[: b.size] = b
    blocks[:, 0] = _bits(torch.tensor([lead], dtype=torch.bfloat16))[0]
    return _from_bits(blocks)


@pytest.mark.parametrize("lead", [448.0, -448.0])
def test_cache_write_fp8_every_bf16_value(dsa, lead):
    # the lead element fixes amax = 448, so the scale is 1 and every quotient is the value itself:
    # the conversion is checked on all representable inputs, ties and subnormals included
    k = _sweep_blocks(lead)
    T = k.shape[0]
    announce("dsa_cache_write fp8, every bf16 value in [-448, 448], %d blocks, lead %g" % (T, lead))
    _run_fp8(dsa, k, np.arange(T), 1, T, rows_per_seq=T)


@pytest.mark.parametrize("round_scale", [False, True])
def test_cache_write_fp8_decode_tokens(dsa, round_scale):
    # one token per sequence; magnitudes from 2^-130 (subnormal scales) to 2^120, zero keys,
    # and positions outside [0, S_max) that must be skipped
    T, S_max = 1000, 64
    g = np.random.default_rng(21)
    x = g.standard_normal((T, 128)) * np.exp2(g.uniform(-130, 120, (T, 1)))
    x[::97] = 0.0
    k = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    pos = g.integers(-2, S_max + 2, size=T)
    announce("dsa_cache_write fp8 decode tokens T=%d S_max=%d round_scale=%s" % (T, S_max, round_scale))
    _run_fp8(dsa, k, pos, T, S_max, round_scale=round_scale, seed=1)


def test_cache_write_fp8_prefill_rows(dsa):
    # two sequences of 777 tokens each writing a permutation of 777 of the 1000 slots
    rps, S_max = 777, 1000
    g = np.random.default_rng(22)
    pos = np.concatenate([g.permutation(S_max)[:rps] for _ in range(2)])
    k = synthetic.normal(23, 0, (2 * rps, 128))
    announce("dsa_cache_write fp8 prefill 2 x %d tokens into %d slots" % (rps, S_max))
    _run_fp8(dsa, k, pos, 2, S_max, rows_per_seq=rps, seed=2)


@pytest.mark.parametrize("qdq,round_scale", [(False, False), (True, False), (True, True)])
def test_cache_write_bf16(dsa, qdq, round_scale):
    T, S_max = 333, 50
    g = np.random.default_rng(24)
    x = g.standard_normal((T, 128)) * np.exp2(g.uniform(-60, 60, (T, 1)))
    k = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    pos = g.integers(-1, S_max + 1, size=T)
    cache0 = g.integers(0, 1 << 16, size=(T, S_max, 128), dtype=np.uint32).astype(np.uint16)
    announce("dsa_cache_write bf16 T=%d qdq=%s round_scale=%s" % (T, qdq, round_scale))
    kc = _from_bits(cache0).cuda()
    dsa.dsa_cache_write(k.cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(), kc, qdq=qdq,
                        round_scale=round_scale)
    torch.cuda.synchronize()
    want = oracle.cache_write(k, pos, cache0, qdq=qdq, round_scale=round_scale)
    assert np.array_equal(_bits(kc), want)


def test_cache_write_empty(dsa):
    announce("dsa_cache_write T=0")
    kc = torch.full((1, 8, 128), 7, dtype=torch.uint8, device="cuda")
    ks = torch.ones((1, 8), dtype=torch.float32, device="cuda")
    dsa.dsa_cache_write(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"),
                        torch.empty((0,), dtype=torch.int32, device="cuda"), kc, k_scale=ks, rows_per_seq=1)
    torch.cuda.synchronize()
    assert bool((kc == 7).all()) and bool((ks == 1).all())


def test_cache_write_then_score(dsa):
    """Quantise a whole fp8 cache on the GPU, append one new key per sequence, then score it:
    the scores match the oracle's quantiser followed by the oracle's scorer."""
    M, S_max, H = 3, 3000, 64
    w = synthetic.make_workload("fp8_long_decode", M=M, S_max=S_max, vl_lo=1000, topk=64)
    keys = synthetic.normal(31, 0, (M * S_max, 128))
    pos_all = np.tile(np.arange(S_max), M)
    announce("dsa_cache_write fp8 %d x %d slots, one new key per row, then dsa_index_score" % (M, S_max))
    kc = torch.zeros((M, S_max, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((M, S_max), dtype=torch.float32, device="cuda")
    dsa.dsa_cache_write(keys.cuda(), torch.from_numpy(pos_all.astype(np.int32)).cuda(), kc, k_scale=ks,
                        rows_per_seq=S_max)
    new = synthetic.normal(32, 0, (M, 128)) * 4
    pos = w.positions.numpy()
    dsa.dsa_cache_write(new.cuda(), w.positions.cuda(), kc, k_scale=ks)
    got = dsa.dsa_index_score(w.index_q.cuda(), w.index_w.cuda(), kc, scale=w.index_scale, k_scale=ks,
                              positions=w.positions.cuda())
    torch.cuda.synchronize()
    c0, s0 = oracle.cache_write(keys, pos_all, np.zeros((M, S_max, 128), np.uint8), np.zeros((M, S_max), np.float32),
                                rows_per_seq=S_max)
    c1, s1 = oracle.cache_write(new, pos, c0, s0)
    assert np.array_equal(kc.cpu().numpy(), c1) and np.array_equal(ks.cpu().numpy(), s1)
    ref = oracle.index_score(w.index_q, w.index_w, c1, k_scale=s1, scale=w.index_scale, positions=w.positions)
    from parity import check_scores, n_valid_rows

    nv = n_valid_rows(pos, -1, M, S_max)
    check_scores(got.cpu().numpy(), ref, nv, oracle.mask_bound())
