"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``dsa_oracle.c`` (plain C,
double precision, no code shared with the HIP library) through ctypes and
converts numpy / torch CPU arrays to the raw encodings the C code decodes
itself (float64, bfloat16 bit patterns, OCP FP8 E4M3 codes).

Functions follow the web pages cited in ``dsa_oracle.c``:
  * ``index_score``  -- lightning-indexer scores with the finite mask bound
  * ``topk``         -- full-sort top-k (unordered-set contract), -1 padding
  * ``assemble``     -- top-k plus always-selected sliding window
  * ``sparse_attn``  -- two-pass softmax-with-sink attention over an index list
  * ``masked_dense_attn`` -- the same attention over the set of listed slots,
                        as a dense masked pass over every slot
  * ``n_valid``      -- attendable slots of a row
  * ``quantize_fp8_blocks`` / ``dequantize_fp8_blocks`` -- FP8 E4M3 block
                        quantiser (binary32 decisions, nearest code, ties even)
  * ``cache_write``  -- new keys stored at their positions, optionally quantised
  * ``unpage``       -- a paged pool read back as contiguous per-sequence caches
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F64, BF16, FP8_E4M3 = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c into liboracle.so (gcc, -O2, strict IEEE, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f64, ip = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.oracle_mask_bound.restype = ctypes.c_float
    lib.oracle_n_valid.argtypes = [vp, i32, i64, i32]
    lib.oracle_n_valid.restype = i32
    lib.oracle_decode_bf16.argtypes = [vp, vp, i64]
    lib.oracle_decode_fp8_e4m3.argtypes = [vp, vp, i64]
    lib.oracle_index_score.argtypes = [vp, ip, vp, vp, ip, vp, vp, i32, i32, i32, i32, i32, i32, f64, ip, vp, ip]
    lib.oracle_topk.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, ip]
    lib.oracle_assemble.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp]
    lib.oracle_sparse_attn.argtypes = [vp, ip, vp, ip, vp, vp, i32, i32, i32, i32, i32, i32, i32, f64, vp, vp, ip]
    lib.oracle_masked_dense_attn.argtypes = [vp, ip, vp, ip, vp, vp, i32, i32, i32, i32, i32, i32, i32, f64, vp, vp,
                                             ip]
    lib.oracle_encode_fp8_e4m3.argtypes = [vp, vp, i64]
    lib.oracle_quantize_fp8_blocks.argtypes = [vp, i64, i32, ip, vp, vp]
    lib.oracle_dequantize_fp8_blocks.argtypes = [vp, vp, i64, i32, vp]
    _lib = lib
    return lib


def default_threads() -> int:
    """Every core this process may run on, or OMP_NUM_THREADS when that is set lower (a host that grants
    the process a share of its cores says so there)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and 0 < int(env) < n:
        n = int(env)
    return n


def _raw(x):
    """Return (contiguous numpy array, dtype code) for float64 / bf16 / fp8 inputs.

    Accepted: numpy float64 (F64), numpy uint16 (bfloat16 bit patterns),
    numpy uint8 (FP8 E4M3 codes), or torch CPU tensors of dtype float64,
    bfloat16 or float8_e4m3fn.
    """
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float8_e4m3fn:
                return x.view(torch.uint8).numpy(), FP8_E4M3
            if x.dtype == torch.uint8:
                return x.numpy(), FP8_E4M3
            x = x.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.uint8:
        return x, FP8_E4M3
    return np.ascontiguousarray(x, dtype=np.float64), F64


def _np(x, dtype):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def mask_bound() -> float:
    return float(_load().oracle_mask_bound())


def n_valid(positions, valid_len: int, row: int, s_max: int) -> int:
    pos = _np(positions, np.int32)
    return int(_load().oracle_n_valid(_ptr(pos), int(valid_len), int(row), int(s_max)))


def decode_bf16(bits) -> np.ndarray:
    a = _np(bits, np.uint16)
    out = np.empty(a.shape, np.float64)
    _load().oracle_decode_bf16(_ptr(a), _ptr(out), a.size)
    return out


def decode_fp8_e4m3(codes) -> np.ndarray:
    a = _np(codes, np.uint8)
    out = np.empty(a.shape, np.float64)
    _load().oracle_decode_fp8_e4m3(_ptr(a), _ptr(out), a.size)
    return out


def index_score(q, w, k, *, scale: float, k_scale=None, positions=None, valid_len: int = -1,
                rows_per_seq: int = 1, relu: bool = False, nthreads: int | None = None) -> np.ndarray:
    """Indexer scores [M, S_max] fp32.  q [M, H, D]; w [M, H]; k [M // rows_per_seq, S_max, D]."""
    qa, qt = _raw(q)
    ka, kt = _raw(k)
    wa = _np(w, np.float32)
    M, H, D = qa.shape
    n_seq, S_max, Dk = ka.shape
    assert Dk == D and wa.shape == (M, H) and M % rows_per_seq == 0 and n_seq == M // rows_per_seq
    ks = _np(k_scale, np.float32)
    if kt == FP8_E4M3:
        assert ks is not None and ks.shape == (n_seq, S_max)
    pos = _np(positions, np.int32)
    if pos is not None:
        assert pos.shape == (M,)
    out = np.empty((M, S_max), np.float32)
    _load().oracle_index_score(_ptr(qa), qt, _ptr(wa), _ptr(ka), kt, _ptr(ks), _ptr(pos), int(valid_len),
                               M, rows_per_seq, H, D, S_max, float(scale), int(bool(relu)), _ptr(out),
                               nthreads or default_threads())
    return out


def topk(scores, k: int, *, positions=None, valid_len: int = -1, with_scores: bool = False,
         nthreads: int | None = None):
    """Top-k slot indices [M, k] int32 (sorted by the oracle, a set by contract); -1 padding."""
    sc = _np(scores, np.float32)
    M, S_max = sc.shape
    pos = _np(positions, np.int32)
    idx = np.empty((M, k), np.int32)
    tsc = np.empty((M, k), np.float32) if with_scores else None
    _load().oracle_topk(_ptr(sc), M, S_max, _ptr(pos), int(valid_len), int(k), _ptr(idx), _ptr(tsc),
                        nthreads or default_threads())
    return (idx, tsc) if with_scores else idx


def assemble(topk_idx, *, s_max: int, window: int, positions=None, valid_len: int = -1) -> np.ndarray:
    """Top-k plus sliding window, [B, k + window] int32 (-1 = masked)."""
    t = _np(topk_idx, np.int32)
    B, k = t.shape
    pos = _np(positions, np.int32)
    out = np.empty((B, k + window), np.int32)
    _load().oracle_assemble(_ptr(t), _ptr(pos), int(valid_len), B, int(s_max), k, int(window), _ptr(out))
    return out


def sparse_attn(q, kv, sink, idx, *, sm_scale: float, dv: int, nthreads: int | None = None):
    """Sparse attention with sink.  q [B, S, Hq, Dqk]; kv [B, S_kv, Dqk]; sink [Hq] or None;
    idx [B, S, K_top].  Returns (out [B, S, Hq, dv] float64, lse [B, S, Hq] float64)."""
    qa, qt = _raw(q)
    ka, kt = _raw(kv)
    B, S, Hq, Dqk = qa.shape
    Bk, S_kv, Dk = ka.shape
    assert Bk == B and Dk == Dqk and 0 < dv <= Dqk
    ia = _np(idx, np.int32)
    assert ia.shape[:2] == (B, S)
    K_top = ia.shape[2]
    sk = _np(sink, np.float32)
    if sk is not None:
        assert sk.shape == (Hq,)
    out = np.empty((B, S, Hq, dv), np.float64)
    lse = np.empty((B, S, Hq), np.float64)
    _load().oracle_sparse_attn(_ptr(qa), qt, _ptr(ka), kt, _ptr(sk), _ptr(ia), B, S, Hq, Dqk, dv, S_kv, K_top,
                               float(sm_scale), _ptr(out), _ptr(lse), nthreads or default_threads())
    return out, lse


def masked_dense_attn(q, kv, sink, idx, *, sm_scale: float, dv: int, nthreads: int | None = None):
    """Masked dense attention with sink (OpenXLA tokamax "Supported Ops and Hardware", masked_dense_mla):
    every slot of the sequence, masked unless the list selects it (a slot listed twice counts once).
    Shapes and results as ``sparse_attn``."""
    qa, qt = _raw(q)
    ka, kt = _raw(kv)
    B, S, Hq, Dqk = qa.shape
    Bk, S_kv, Dk = ka.shape
    assert Bk == B and Dk == Dqk and 0 < dv <= Dqk
    ia = _np(idx, np.int32)
    assert ia.shape[:2] == (B, S)
    K_top = ia.shape[2]
    sk = _np(sink, np.float32)
    if sk is not None:
        assert sk.shape == (Hq,)
    out = np.empty((B, S, Hq, dv), np.float64)
    lse = np.empty((B, S, Hq), np.float64)
    _load().oracle_masked_dense_attn(_ptr(qa), qt, _ptr(ka), kt, _ptr(sk), _ptr(ia), B, S, Hq, Dqk, dv, S_kv, K_top,
                                     float(sm_scale), _ptr(out), _ptr(lse), nthreads or default_threads())
    return out, lse


# ------------------------------------------------------------ key-cache write

QUANT_BLOCK = 128  # elements per FP8 quantisation block ([V4-KERNEL] FP8 block quantisation)


def _bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of a torch bfloat16 tensor or a uint16 array."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            assert x.dtype == torch.bfloat16
            return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    assert a.dtype == np.uint16
    return a


def encode_fp8_e4m3(y) -> np.ndarray:
    """Nearest E4M3 codes (ties to even) of binary32 values with |y| <= 448."""
    a = _np(y, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().oracle_encode_fp8_e4m3(_ptr(a), _ptr(out), a.size)
    return out


def quantize_fp8_blocks(x, *, round_scale: bool = False, block: int = QUANT_BLOCK):
    """FP8 block quantisation of bfloat16 x [..., D] (D a multiple of block).

    Returns (codes uint8 [..., D], scales float32 [..., D // block])."""
    bits = _bf16_bits(x)
    D = bits.shape[-1]
    assert D % block == 0
    n_blocks = bits.size // block
    codes = np.empty(bits.shape, np.uint8)
    scales = np.empty(bits.shape[:-1] + (D // block,), np.float32)
    _load().oracle_quantize_fp8_blocks(_ptr(bits), n_blocks, block, int(bool(round_scale)), _ptr(codes),
                                       _ptr(scales))
    return codes, scales


def dequantize_fp8_blocks(codes, scales, *, block: int = QUANT_BLOCK) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of value(code) * scale, rounded once."""
    c = _np(codes, np.uint8)
    sc = _np(scales, np.float32)
    assert c.shape[-1] % block == 0 and sc.size * block == c.size
    out = np.empty(c.shape, np.uint16)
    _load().oracle_dequantize_fp8_blocks(_ptr(c), _ptr(sc), c.size // block, block, _ptr(out))
    return out


def cache_write(k_new, positions, k_cache, k_scale=None, *, rows_per_seq: int = 1, round_scale: bool = False,
                qdq: bool = False):
    """Key-cache write: token t of k_new [T, D] (bfloat16) goes to cache row
    t // rows_per_seq at slot positions[t], in place at the token's position
    ([NKI-V32] key_cache); tokens whose position is outside [0, S_max) are
    not written.

    * FP8 cache (``k_cache`` uint8 codes [n_seq, S_max, D] with ``k_scale``
      float32 [n_seq, S_max, D // 128]): the key is block-quantised.
    * bfloat16 cache (bit patterns uint16 or a bfloat16 tensor): the key is
      stored as is, or with ``qdq`` quantised and dequantised back.

    Returns updated copies (numpy): (codes, scales) or the bfloat16 bits."""
    kb = _bf16_bits(k_new)
    T, D = kb.shape
    pos = _np(positions, np.int32)
    assert pos.shape == (T,) and T % rows_per_seq == 0
    fp8 = k_scale is not None
    if fp8:
        cache = np.array(_np(k_cache, np.uint8))
        scales = np.array(_np(k_scale, np.float32))
        codes, sc = quantize_fp8_blocks(kb, round_scale=round_scale)
    else:
        cache = np.array(_bf16_bits(k_cache))
        if qdq:
            codes, sc = quantize_fp8_blocks(kb, round_scale=round_scale)
            vals = dequantize_fp8_blocks(codes, sc)
        else:
            vals = kb
    n_seq, S_max, Dc = cache.shape
    assert Dc == D and n_seq == T // rows_per_seq
    for t in range(T):
        c, p = t // rows_per_seq, int(pos[t])
        if not 0 <= p < S_max:
            continue
        if fp8:
            cache[c, p] = codes[t]
            scales[c, p] = sc[t].reshape(scales[c, p].shape)
        else:
            cache[c, p] = vals[t]
    return (cache, scales) if fp8 else cache


# ------------------------------------------------------------- paged caches

def unpage(pool, block_table, page_size: int, n_slots: int) -> np.ndarray:
    """Contiguous [n_seq, n_slots, ...] view of a page pool [n_pages * page_size, ...]: slot s of
    sequence r is pool row block_table[r, s // page_size] * page_size + s % page_size
    (tokamax "Supported Ops and Hardware", lightning_indexer over a paged KV cache)."""
    try:
        import torch

        if isinstance(pool, torch.Tensor):
            pool = pool.detach().cpu()
            if pool.dtype == torch.bfloat16:
                pool = pool.view(torch.int16).numpy().view(np.uint16)
            elif pool.dtype == torch.float8_e4m3fn:
                pool = pool.view(torch.uint8).numpy()
            else:
                pool = pool.numpy()
    except ImportError:  # pragma: no cover
        pass
    bt = _np(block_table, np.int64)
    n_seq = bt.shape[0]
    out = np.empty((n_seq, n_slots) + pool.shape[1:], pool.dtype)
    for r in range(n_seq):
        for s in range(0, n_slots, page_size):
            n = min(page_size, n_slots - s)
            base = bt[r, s // page_size] * page_size
            out[r, s:s + n] = pool[base:base + n]
    return out
