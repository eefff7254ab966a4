"""The C-ABI library loads, exports every symbol include/dsa.h declares, and
validates arguments on the host (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_amd", "libdsa.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    import sparse_attention_amd as m

    return m.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dsa_index_score", "dsa_topk", "dsa_sparse_attn", "dsa_decode_step"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_constants(lib):
    assert lib.dsa_version().decode().count(".") == 2
    mb = lib.dsa_mask_bound()
    import struct
    assert struct.unpack("<I", struct.pack("<f", mb))[0] == 0xFF7F0000
    assert b"NULL" in lib.dsa_status_string(ERR_NULL)


def _p(v):
    return ctypes.c_void_p(v)


A = 0x10000  # a fake, aligned, non-null "device" address; never dereferenced on these paths


def test_index_score_validation(lib):
    f = lib.dsa_index_score
    args = dict(q=_p(A), w=_p(A), k=_p(A), ks=None, kd=0, pos=None, vl=-1, M=2, rps=1, H=4, D=128, S=100,
                scale=1.0, flags=0, out=_p(A))

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["w"], a["k"], a["ks"], a["kd"], a["pos"], a["vl"], a["M"], a["rps"], a["H"], a["D"],
                 a["S"], a["scale"], a["flags"], a["out"], None)

    assert call(q=None) == ERR_NULL
    assert call(out=None) == ERR_NULL
    assert call(kd=1) == ERR_NULL                 # fp8 without scales
    assert call(ks=_p(A)) == ERR_SHAPE            # bf16 with scales
    assert call(D=64) == ERR_UNSUPPORTED
    assert call(H=0) == ERR_SHAPE
    assert call(H=129) == ERR_UNSUPPORTED
    assert call(M=3, rps=2) == ERR_SHAPE
    assert call(flags=1, H=65) == ERR_UNSUPPORTED  # relu decode: per-head path, at most 64 heads
    assert call(flags=4) == ERR_UNSUPPORTED
    assert call(q=_p(A + 8)) == ERR_ALIGN
    assert call(kd=7) == ERR_UNSUPPORTED
    # prefill (rows_per_seq > 1): bf16 keys; the per-head MFMA path (ReLU) takes at most 64 heads
    assert call(M=4, rps=4, H=65, flags=1) == ERR_UNSUPPORTED
    assert call(M=4, rps=4, kd=1, ks=_p(A)) == ERR_UNSUPPORTED


def test_topk_validation(lib):
    f = lib.dsa_topk
    assert f(None, 1, 10, None, -1, 4, _p(A), None, None, 0, None) == ERR_NULL
    assert f(_p(A), 0, 10, None, -1, 4, _p(A), None, None, 0, None) == ERR_SHAPE
    assert f(_p(A), 1, 10, None, -1, 0, _p(A), None, None, 0, None) == ERR_UNSUPPORTED
    assert f(_p(A), 1, 10, None, -1, 2049, _p(A), None, None, 0, None) == ERR_UNSUPPORTED
    need = lib.dsa_topk_workspace_size(16, 32768, 1024)
    assert need >= 16 * 32768 * 4
    assert f(_p(A), 16, 32768, None, -1, 1024, _p(A), None, None, 0, None) == ERR_WORKSPACE
    assert f(_p(A), 16, 32768, None, -1, 1024, _p(A), None, _p(A), need - 1, None) == ERR_WORKSPACE
    assert f(_p(A), 16, 32768, None, -1, 1024, _p(A), None, _p(A + 8), need, None) == ERR_ALIGN
    assert lib.dsa_topk_workspace_size(8192, 8192, 2048) == 0  # many short rows: one workgroup per row


def test_masked_dense_attn_validation_and_workspace(lib):
    f = lib.dsa_sparse_attn_masked_dense
    need = lib.dsa_sparse_attn_masked_dense_workspace_size(2, 1, 128, 512, 4096)
    # the dense slot list of each token, then the partials of a 4096-entry list
    assert need >= 2 * 4096 * 4 + lib.dsa_sparse_attn_workspace_size(2, 1, 128, 512, 4096)

    def call(S_kv=4096, K=64, Dv=512, ws=_p(A), nws=need, q=_p(A)):
        return f(q, _p(A), None, _p(A), 2, 1, 128, 576, Dv, S_kv, K, 0.1, _p(A), None, ws, nws, None)

    assert call(q=None) == ERR_NULL
    assert call(Dv=528) == ERR_UNSUPPORTED
    assert call(K=0) == ERR_SHAPE
    assert call(S_kv=65537) == ERR_SHAPE
    assert lib.dsa_sparse_attn_masked_dense_workspace_size(2, 1, 128, 512, 65537) == 0
    assert call(ws=None, nws=0) == ERR_WORKSPACE
    assert call(nws=need - 1) == ERR_WORKSPACE
    assert call(ws=_p(A + 8)) == ERR_ALIGN


def test_sparse_attn_validation_and_workspace(lib):
    f = lib.dsa_sparse_attn

    def call(B=2, S=1, Hq=128, Dqk=576, Dv=512, S_kv=1000, K=1152, ws=None, nws=0, q=_p(A)):
        return f(q, _p(A), None, _p(A), B, S, Hq, Dqk, Dv, S_kv, K, 0.1, _p(A), None, ws, nws, None)

    assert call(q=None) == ERR_NULL
    assert call(Dqk=600) == ERR_UNSUPPORTED
    assert call(Dqk=100) == ERR_UNSUPPORTED
    assert call(Dv=600) == ERR_UNSUPPORTED
    assert call(Dv=24) == ERR_UNSUPPORTED
    assert call(K=0) == ERR_SHAPE
    # Value features above 512 are rejected (the attention kernels' accumulators hold at most 512)
    assert call(Dqk=576, Dv=528) == ERR_UNSUPPORTED
    assert call(Dqk=576, Dv=576) == ERR_UNSUPPORTED
    # Few tokens: the index list is split over workgroups and the partial
    # results (bf16 output per split + fp32 max and sum) live in the workspace.
    # 2 tokens x 2 head groups -> 8 splits (36 blocks of 32 entries, >= 4 per split)
    need = lib.dsa_sparse_attn_workspace_size(2, 1, 128, 512, 1152)
    assert need == 2 * 8 * 128 * 512 * 2 + 2 * 8 * 128 * 8
    # 64 decode tokens x 2 head groups -> 2 splits
    assert lib.dsa_sparse_attn_workspace_size(64, 1, 128, 512, 1152) == 64 * 2 * 128 * 512 * 2 + 64 * 2 * 128 * 8
    # 256 tokens fill the chip with 128-head workgroups: the other kernel, no split, no workspace
    assert lib.dsa_sparse_attn_workspace_size(256, 1, 128, 512, 1152) == 0
    # enough tokens to fill the chip: no split, no workspace
    assert lib.dsa_sparse_attn_workspace_size(1024, 1, 64, 512, 64) == 0
    # a short list (2 blocks) is not split
    assert lib.dsa_sparse_attn_workspace_size(8, 1, 128, 512, 64) == 0
    assert call() == ERR_WORKSPACE
    assert call(ws=_p(A), nws=need - 1) == ERR_WORKSPACE
    assert call(B=70000) == ERR_SHAPE


def test_decode_step_validation(lib):
    import sparse_attention_amd as m

    a = m._DecodeArgs()
    a.struct_size = ctypes.sizeof(m._DecodeArgs)
    for name in ("index_q", "index_w", "k_cache", "q", "kv", "out"):
        setattr(a, name, A)
    a.B, a.H, a.S_max, a.index_topk, a.window = 4, 64, 4096, 1024, 128
    a.Hq, a.Dqk, a.Dv, a.valid_len = 128, 576, 512, -1
    ws = lib.dsa_decode_step_workspace_size(ctypes.byref(a))
    assert ws >= 4 * 4096 * 4 + 4 * 1152 * 4
    assert lib.dsa_decode_step(ctypes.byref(a), None, 0, None) == ERR_WORKSPACE
    a.window = -1
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_SHAPE
    a.window = 128
    a.q = None
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_NULL
    a.q = A
    a.index_flags = 1
    a.H = 65
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_UNSUPPORTED  # relu: at most 64 heads
    a.H = 64
    a.index_flags = 2
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_UNSUPPORTED  # unknown flag
    a.index_flags = 0
    a.struct_size = 8
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_UNSUPPORTED
    # a struct without index_flags is still accepted: flags read as 0, paging as NULL
    old = m._DecodeArgs.index_flags.offset
    a.struct_size = old
    a.index_flags = 2                      # beyond the given size: ignored
    a.paging = 8                           # (would be an invalid pointer)
    a.window = -1
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_SHAPE  # validation went on past the size
    a.window = 128
    assert lib.dsa_decode_step_workspace_size(ctypes.byref(a)) == ws
    a.window = -1
    # a struct that ends after index_flags but before paging: paging reads as NULL
    a.index_flags = 0
    a.struct_size = m._DecodeArgs.paging.offset
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_SHAPE
    # paged: the descriptor is validated
    a.struct_size = ctypes.sizeof(m._DecodeArgs)
    a.window = 128
    pg = m._PagedCache(A, 64, 64, 1000)  # 64 pages of 64 slots = 4096 = S_max
    a.paging = ctypes.addressof(pg)
    assert lib.dsa_decode_step(ctypes.byref(a), None, 0, None) == ERR_WORKSPACE  # valid up to the workspace
    pg.max_pages = 63
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_SHAPE  # 63 * 64 < S_max
    pg.max_pages, pg.page_size = 64, 96
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_UNSUPPORTED  # not a power of two
    pg.page_size, pg.block_table = 64, None
    assert lib.dsa_decode_step(ctypes.byref(a), _p(A), ws, None) == ERR_NULL


def test_decode_step_static_validation(lib):
    """The allocation-free decode step validates like dsa_decode_step and rejects shapes whose
    scratch exceeds the library's array before touching any device."""
    import sparse_attention_amd as m

    assert lib.dsa_decode_step_static(None, None) == ERR_NULL
    a = m._DecodeArgs()
    a.struct_size = ctypes.sizeof(m._DecodeArgs)
    for name in ("index_q", "index_w", "k_cache", "q", "kv", "out"):
        setattr(a, name, A)
    a.B, a.H, a.S_max, a.index_topk, a.window = 4, 64, 4096, 1024, 128
    a.Hq, a.Dqk, a.Dv, a.valid_len = 128, 576, 512, -1
    a.window = -1
    assert lib.dsa_decode_step_static(ctypes.byref(a), None) == ERR_SHAPE
    a.window, a.Dv = 128, 528
    assert lib.dsa_decode_step_static(ctypes.byref(a), None) == ERR_UNSUPPORTED
    a.Dv, a.q = 512, None
    assert lib.dsa_decode_step_static(ctypes.byref(a), None) == ERR_NULL
    a.q = A
    # 1024 sequences x 65536 slots with scores and list kept in scratch: beyond the 128 MiB array
    a.B, a.S_max = 1024, 65536
    assert lib.dsa_decode_step_workspace_size(ctypes.byref(a)) > m.DSA_STATIC_SCRATCH_BYTES
    assert lib.dsa_decode_step_static(ctypes.byref(a), None) == ERR_WORKSPACE
    # the full decode step shape (64 x 65536, scores kept in scratch) fits
    a.B = 64
    assert lib.dsa_decode_step_workspace_size(ctypes.byref(a)) <= m.DSA_STATIC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert re.search(r"#define DSA_STATIC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", text)
    assert m.DSA_STATIC_SCRATCH_BYTES == 128 << 20


def test_paged_validation(lib):
    import sparse_attention_amd as m

    pg = m._PagedCache(A, 8, 512, 100)
    P = ctypes.byref(pg)
    f = lib.dsa_index_score_paged

    def score(paging=P, **kw):
        a = dict(dict(ks=None, kd=0, M=2, H=4, D=128, S=4096, flags=0), **kw)
        return f(_p(A), _p(A), _p(A), a["ks"], a["kd"], paging, None, -1, a["M"], a["H"], a["D"], a["S"], 1.0,
                 a["flags"], _p(A), None)

    assert score(paging=None) == ERR_NULL
    assert score(S=4097) == ERR_SHAPE          # beyond max_pages * page_size
    assert score(D=64) == ERR_UNSUPPORTED
    assert score(flags=1, H=65) == ERR_UNSUPPORTED
    pg.page_size = 32
    assert score(S=256) == ERR_UNSUPPORTED     # pages below 64 slots
    pg.page_size, pg.n_pages = 512, 1 << 22
    assert score() == ERR_SHAPE                # pool rows beyond 2^31
    pg.n_pages, pg.max_pages = 100, 0
    assert score() == ERR_SHAPE
    pg.max_pages = 8
    g = lib.dsa_sparse_attn_paged

    def attn(paging=P, **kw):
        a = dict(dict(B=2, S=1, Hq=16, Dqk=576, Dv=512, S_kv=4096, K=64), **kw)
        return g(_p(A), _p(A), None, _p(A), paging, a["B"], a["S"], a["Hq"], a["Dqk"], a["Dv"], a["S_kv"], a["K"],
                 0.1, _p(A), None, _p(A), 1 << 30, None)

    assert attn(paging=None) == ERR_NULL
    assert attn(S_kv=4097) == ERR_SHAPE
    assert attn(Dqk=100) == ERR_UNSUPPORTED
    pg.block_table = A + 4
    assert attn() == ERR_ALIGN


def test_cache_write_validation(lib):
    f = lib.dsa_cache_write
    args = dict(k=_p(A), T=4, rps=1, D=128, pos=_p(A), kd=1, kc=_p(A), ks=_p(A), S=100, flags=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["k"], a["T"], a["rps"], a["D"], a["pos"], a["kd"], a["kc"], a["ks"], a["S"], a["flags"], None)

    assert call(k=None) == ERR_NULL
    assert call(pos=None) == ERR_NULL
    assert call(kc=None) == ERR_NULL
    assert call(ks=None) == ERR_NULL               # fp8 without scales
    assert call(kd=0) == ERR_SHAPE                 # bf16 with scales
    assert call(kd=5) == ERR_UNSUPPORTED
    assert call(T=-1) == ERR_SHAPE
    assert call(T=5, rps=2) == ERR_SHAPE
    assert call(rps=0) == ERR_SHAPE
    assert call(S=0) == ERR_SHAPE
    assert call(D=256) == ERR_UNSUPPORTED
    assert call(flags=4) == ERR_UNSUPPORTED
    assert call(flags=2) == ERR_UNSUPPORTED        # quantise-dequantise needs a bf16 cache
    assert call(kd=0, ks=None, flags=1) == ERR_UNSUPPORTED  # a plain bf16 copy computes no scale
    assert call(k=_p(A + 8)) == ERR_ALIGN
    assert call(pos=_p(A + 4)) == ERR_ALIGN
    assert call(T=0) == OK                         # nothing to write: nothing is enqueued
    assert call(T=0, k=None, pos=None) == OK       # (empty tensors may have no storage)


def test_cache_write_paged_validation(lib):
    import sparse_attention_amd as m

    pg = m._PagedCache(A, 4, 64, 100)
    f = lib.dsa_cache_write_paged

    def call(paging=ctypes.byref(pg), **kw):
        a = dict(dict(T=4, rps=1, D=128, kd=1, ks=_p(A), S=256, flags=0), **kw)
        return f(_p(A), a["T"], a["rps"], a["D"], _p(A), a["kd"], _p(A), a["ks"], paging, a["S"], a["flags"], None)

    assert call(paging=None) == ERR_NULL
    assert call(S=257) == ERR_SHAPE            # beyond max_pages * page_size
    assert call(ks=None) == ERR_NULL
    assert call(flags=2) == ERR_UNSUPPORTED
    pg.page_size = 48
    assert call() == ERR_UNSUPPORTED

