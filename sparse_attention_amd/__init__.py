"""Python binding of libdsa, the MI355X (gfx950) DeepSeek Sparse Attention hot path.

Thin ctypes marshalling over the C ABI declared in ``include/dsa.h``: each
function takes torch tensors on the current HIP device, allocates outputs
(and the workspace) with torch, and calls the C entry point of the same name
on ``torch.cuda.current_stream()``.  Every step of the computation runs in
the library's HIP kernels; there is no other code path.  If ``libdsa.so``
has not been built (``python -m sparse_attention_amd.build_lib``) every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_KEY_BF16 = 0
DSA_KEY_FP8_E4M3 = 1
DSA_SCORE_RELU = 1
DSA_CACHE_ROUND_SCALE = 1
DSA_CACHE_QDQ = 2

_STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_UNSUPPORTED", 4: "DSA_ERR_ALIGN",
           5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_LAUNCH"}


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status
        self.status_name = _STATUS.get(status, str(status))


class _DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("index_q", ctypes.c_void_p), ("index_w", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("k_dtype", ctypes.c_int), ("positions", ctypes.c_void_p),
        ("valid_len", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S_max", ctypes.c_int32),
        ("index_scale", ctypes.c_float), ("index_topk", ctypes.c_int32), ("window", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("attn_sink", ctypes.c_void_p),
        ("Hq", ctypes.c_int32), ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("scores", ctypes.c_void_p),
        ("index_list", ctypes.c_void_p), ("index_flags", ctypes.c_uint32), ("paging", ctypes.c_void_p),
    ]


class _PagedCache(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


class Paging:
    """A paged cache layout: block_table [n_seq, max_pages] int32 on the GPU, page_size slots per page,
    n_pages pages in the pool.  Pools are [n_pages * page_size, ...] tensors."""

    def __init__(self, block_table: torch.Tensor, page_size: int, n_pages: int):
        _dev(block_table, "block_table", (torch.int32,))
        self.block_table = block_table
        self.page_size, self.n_pages = int(page_size), int(n_pages)
        self.struct = _PagedCache(block_table.data_ptr(), int(block_table.shape[1]), self.page_size, self.n_pages)


_lib = None


def load_library(path: Optional[str] = None):
    """Load libdsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libdsa.so not found at %s: build it with `python -m sparse_attention_amd.build_lib`" % p)
    lib = ctypes.CDLL(p)
    vp, i32, f32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint32, ctypes.c_size_t
    st = ctypes.c_int
    lib.dsa_version.restype = ctypes.c_char_p
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_status_string.argtypes = [st]
    lib.dsa_mask_bound.restype = f32
    lib.dsa_index_score.restype = st
    lib.dsa_index_score.argtypes = [vp, vp, vp, vp, st, vp, i32, i32, i32, i32, i32, i32, f32, u32, vp, vp]
    lib.dsa_topk_workspace_size.restype = sz
    lib.dsa_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_topk.restype = st
    lib.dsa_topk.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.dsa_sparse_attn_workspace_size.restype = sz
    lib.dsa_sparse_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.dsa_sparse_attn.restype = st
    lib.dsa_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.dsa_sparse_attn_masked_dense_workspace_size.restype = sz
    lib.dsa_sparse_attn_masked_dense_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.dsa_sparse_attn_masked_dense.restype = st
    lib.dsa_sparse_attn_masked_dense.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                                 sz, vp]
    lib.dsa_decode_step_workspace_size.restype = sz
    lib.dsa_decode_step_workspace_size.argtypes = [ctypes.POINTER(_DecodeArgs)]
    lib.dsa_decode_step.restype = st
    lib.dsa_decode_step.argtypes = [ctypes.POINTER(_DecodeArgs), vp, sz, vp]
    lib.dsa_decode_step_static.restype = st
    lib.dsa_decode_step_static.argtypes = [ctypes.POINTER(_DecodeArgs), vp]
    pp = ctypes.POINTER(_PagedCache)
    lib.dsa_index_score_paged.restype = st
    lib.dsa_index_score_paged.argtypes = [vp, vp, vp, vp, st, pp, vp, i32, i32, i32, i32, i32, f32, u32, vp, vp]
    lib.dsa_sparse_attn_paged.restype = st
    lib.dsa_sparse_attn_paged.argtypes = [vp, vp, vp, vp, pp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, sz,
                                          vp]
    lib.dsa_cache_write_paged.restype = st
    lib.dsa_cache_write_paged.argtypes = [vp, i32, i32, i32, vp, st, vp, vp, pp, i32, u32, vp]
    lib.dsa_cache_write.restype = st
    lib.dsa_cache_write.argtypes = [vp, i32, i32, i32, vp, st, vp, vp, i32, u32, vp]
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = load_library().dsa_status_string(status).decode()
        raise DsaError(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a tensor on the GPU" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def version() -> str:
    return load_library().dsa_version().decode()


def mask_bound() -> float:
    return float(load_library().dsa_mask_bound())


def _key_args(k_cache: torch.Tensor, k_scale: Optional[torch.Tensor]):
    if k_cache.dtype == torch.bfloat16:
        return DSA_KEY_BF16
    _dev(k_scale, "k_scale", (torch.float32,)) if k_scale is not None else None
    return DSA_KEY_FP8_E4M3


def dsa_index_score(q, w, k_cache, *, scale: float, k_scale=None, positions=None, valid_len: int = -1,
                    rows_per_seq: int = 1, relu: bool = False, out=None, paging: Optional[Paging] = None,
                    s_max: Optional[int] = None) -> torch.Tensor:
    """Indexer scores [M, S_max] fp32.  q [M, H, 128] bf16; w [M, H] fp32;
    k_cache [M // rows_per_seq, S_max, 128] bf16 or uint8/float8_e4m3fn codes (+ k_scale [n_seq, S_max]).
    With ``paging`` (decode rows only), k_cache / k_scale are page pools [n_pages * page_size, ...] and
    ``s_max`` is the logical slot count of every sequence."""
    _dev(q, "q", (torch.bfloat16,))
    _dev(w, "w", (torch.float32,))
    _dev(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn))
    kd = _key_args(k_cache, k_scale)
    if positions is not None:
        _dev(positions, "positions", (torch.int32,))
    M, H, D = q.shape
    if paging is not None:
        if s_max is None or rows_per_seq != 1:
            raise ValueError("paged scoring needs s_max and one row per sequence")
        S_max = int(s_max)
    else:
        S_max = k_cache.shape[1]
    if out is None:
        out = torch.empty((M, S_max), dtype=torch.float32, device=q.device)
    _dev(out, "out", (torch.float32,))
    flags = DSA_SCORE_RELU if relu else 0
    lib = load_library()
    if paging is not None:
        st = lib.dsa_index_score_paged(_ptr(q), _ptr(w), _ptr(k_cache), _ptr(k_scale), kd, ctypes.byref(paging.struct),
                                       _ptr(positions), int(valid_len), M, H, D, S_max, float(scale), flags, _ptr(out),
                                       _stream())
        _check("dsa_index_score_paged", st)
        return out
    st = lib.dsa_index_score(_ptr(q), _ptr(w), _ptr(k_cache), _ptr(k_scale), kd, _ptr(positions), int(valid_len), M,
                             int(rows_per_seq), H, D, S_max, float(scale), flags, _ptr(out), _stream())
    _check("dsa_index_score", st)
    return out


def topk_workspace_bytes(M: int, S_max: int, index_topk: int) -> int:
    return int(load_library().dsa_topk_workspace_size(int(M), int(S_max), int(index_topk)))


def dsa_topk(scores, index_topk: int, *, positions=None, valid_len: int = -1, with_scores: bool = False,
             out=None, workspace=None):
    """Top-k slot indices [M, index_topk] int32 (unordered set per row, -1 padded; the same scores give
    the same row on every call).  ``out`` and ``workspace`` (uint8, at least topk_workspace_bytes) may be
    given to avoid allocations."""
    _dev(scores, "scores", (torch.float32,))
    if positions is not None:
        _dev(positions, "positions", (torch.int32,))
    M, S_max = scores.shape
    lib = load_library()
    idx = out if out is not None else torch.empty((M, index_topk), dtype=torch.int32, device=scores.device)
    _dev(idx, "out", (torch.int32,))
    if tuple(idx.shape) != (M, index_topk):
        raise ValueError("out must be [M, index_topk]")
    tsc = torch.empty((M, index_topk), dtype=torch.float32, device=scores.device) if with_scores else None
    nws = lib.dsa_topk_workspace_size(M, S_max, int(index_topk))
    ws = workspace if workspace is not None else _workspace(nws, scores.device)
    if nws and (ws is None or ws.numel() * ws.element_size() < nws):
        raise ValueError("workspace must hold %d bytes" % nws)
    st = lib.dsa_topk(_ptr(scores), M, S_max, _ptr(positions), int(valid_len), int(index_topk), _ptr(idx), _ptr(tsc),
                      _ptr(ws), nws, _stream())
    _check("dsa_topk", st)
    return (idx, tsc) if with_scores else idx


def sparse_attn_workspace_bytes(B: int, S: int, Hq: int, dv: int, K_top: int) -> int:
    return int(load_library().dsa_sparse_attn_workspace_size(int(B), int(S), int(Hq), int(dv), int(K_top)))


def dsa_sparse_attn(q, kv, attn_sink, topk_idx, *, sm_scale: float, dv: int, with_lse: bool = False, out=None,
                    paging: Optional[Paging] = None, s_kv: Optional[int] = None, workspace=None):
    """Sparse MQA with sink.  q [B, S, Hq, Dqk] bf16; kv [B, S_kv, Dqk] bf16; attn_sink [Hq] fp32 or None;
    topk_idx [B, S, K_top] int32.  Returns out [B, S, Hq, dv] bf16 (and lse [B, S, Hq] fp32); `out` may be
    given, and so may ``workspace`` (uint8, at least sparse_attn_workspace_bytes).  With ``paging``, kv is a
    page pool [n_pages * page_size, Dqk] and ``s_kv`` the logical slot count of every sequence."""
    _dev(q, "q", (torch.bfloat16,))
    _dev(kv, "kv", (torch.bfloat16,))
    _dev(topk_idx, "topk_idx", (torch.int32,))
    if attn_sink is not None:
        _dev(attn_sink, "attn_sink", (torch.float32,))
    B, S, Hq, Dqk = q.shape
    if paging is not None and s_kv is None:
        raise ValueError("paged attention needs s_kv")
    S_kv = int(s_kv) if paging is not None else kv.shape[1]
    K_top = topk_idx.shape[2]
    lib = load_library()
    if out is None:
        out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,))
    if tuple(out.shape) != (B, S, Hq, dv):
        raise ValueError("out must be [B, S, Hq, dv]")
    lse = torch.empty((B, S, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    nws = lib.dsa_sparse_attn_workspace_size(B, S, Hq, int(dv), K_top)
    ws = workspace if workspace is not None else _workspace(nws, q.device)
    if nws and (ws is None or ws.numel() * ws.element_size() < nws):
        raise ValueError("workspace must hold %d bytes" % nws)
    if paging is not None:
        st = lib.dsa_sparse_attn_paged(_ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idx), ctypes.byref(paging.struct),
                                       B, S, Hq, Dqk, int(dv), S_kv, K_top, float(sm_scale), _ptr(out), _ptr(lse),
                                       _ptr(ws), nws, _stream())
        _check("dsa_sparse_attn_paged", st)
    else:
        st = lib.dsa_sparse_attn(_ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idx), B, S, Hq, Dqk, int(dv), S_kv,
                                 K_top, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), nws, _stream())
        _check("dsa_sparse_attn", st)
    return (out, lse) if with_lse else out


def dsa_sparse_attn_masked_dense(q, kv, attn_sink, topk_idx, *, sm_scale: float, dv: int, with_lse: bool = False,
                                 out=None, workspace=None):
    """The attention of dsa_sparse_attn over the set of listed slots, computed densely over all S_kv slots
    (a slot listed twice counts once).  Arguments and results as dsa_sparse_attn; ``workspace`` (uint8, at
    least masked_dense_workspace_bytes) may be given to avoid an allocation."""
    _dev(q, "q", (torch.bfloat16,))
    _dev(kv, "kv", (torch.bfloat16,))
    _dev(topk_idx, "topk_idx", (torch.int32,))
    if attn_sink is not None:
        _dev(attn_sink, "attn_sink", (torch.float32,))
    B, S, Hq, Dqk = q.shape
    S_kv = kv.shape[1]
    K_top = topk_idx.shape[2]
    lib = load_library()
    if out is None:
        out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,))
    if tuple(out.shape) != (B, S, Hq, dv):
        raise ValueError("out must be [B, S, Hq, dv]")
    lse = torch.empty((B, S, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    nws = lib.dsa_sparse_attn_masked_dense_workspace_size(B, S, Hq, int(dv), S_kv)
    ws = workspace if workspace is not None else _workspace(nws, q.device)
    if nws and (ws is None or ws.numel() * ws.element_size() < nws):
        raise ValueError("workspace must hold %d bytes" % nws)
    st = lib.dsa_sparse_attn_masked_dense(_ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idx), B, S, Hq, Dqk,
                                          int(dv), S_kv, K_top, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), nws,
                                          _stream())
    _check("dsa_sparse_attn_masked_dense", st)
    return (out, lse) if with_lse else out


def masked_dense_workspace_bytes(B: int, S: int, Hq: int, dv: int, S_kv: int) -> int:
    return int(load_library().dsa_sparse_attn_masked_dense_workspace_size(int(B), int(S), int(Hq), int(dv),
                                                                          int(S_kv)))


DSA_STATIC_SCRATCH_BYTES = 128 << 20


class DecodeStep:
    """Reusable dsa_decode_step call: validates shapes once, owns the workspace and outputs.

    With ``static_scratch`` the step calls dsa_decode_step_static instead: no workspace is allocated and the
    library's per-GPU scratch array (DSA_STATIC_SCRATCH_BYTES) is used; calls on one GPU must not overlap.

    With ``graph`` the first call runs the step once and captures it into a HIP graph (the library issues only
    kernel launches on the caller's stream: no allocation, memset or synchronisation), and every later call
    replays that graph: one host call per step instead of one kernel launch per stage.  The graph reads and
    writes the buffers given here, so new inputs are written into them in place (as a serving loop does with
    its caches and query buffers)."""

    def __init__(self, index_q, index_w, k_cache, *, positions=None, valid_len: int = -1, index_scale: float,
                 index_topk: int, window: int, q, kv, attn_sink, sm_scale: float, dv: int, k_scale=None,
                 keep_scores: bool = True, keep_index_list: bool = True, relu: bool = False,
                 paging: Optional[Paging] = None, s_max: Optional[int] = None, static_scratch: bool = False,
                 graph: bool = False):
        _dev(index_q, "index_q", (torch.bfloat16,))
        _dev(index_w, "index_w", (torch.float32,))
        _dev(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn))
        _dev(q, "q", (torch.bfloat16,))
        _dev(kv, "kv", (torch.bfloat16,))
        if positions is not None:
            _dev(positions, "positions", (torch.int32,))
        if attn_sink is not None:
            _dev(attn_sink, "attn_sink", (torch.float32,))
        kd = _key_args(k_cache, k_scale)
        B, H, _ = index_q.shape
        if paging is not None and s_max is None:
            raise ValueError("a paged decode step needs s_max")
        S_max = int(s_max) if paging is not None else k_cache.shape[1]
        _, S, Hq, Dqk = q.shape
        if S != 1:
            raise ValueError("decode step takes one query token per sequence")
        dev = q.device
        self.out = torch.empty((B, 1, Hq, dv), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, S_max), dtype=torch.float32, device=dev) if keep_scores else None
        self.index_list = (torch.empty((B, index_topk + window), dtype=torch.int32, device=dev)
                           if keep_index_list else None)
        self._keep = (index_q, index_w, k_cache, k_scale, positions, q, kv, attn_sink, paging)
        a = _DecodeArgs()
        a.struct_size = ctypes.sizeof(_DecodeArgs)
        a.index_q, a.index_w, a.k_cache = index_q.data_ptr(), index_w.data_ptr(), k_cache.data_ptr()
        a.k_scale = None if k_scale is None else k_scale.data_ptr()
        a.k_dtype = kd
        a.positions = None if positions is None else positions.data_ptr()
        a.valid_len, a.B, a.H, a.S_max = int(valid_len), B, H, S_max
        a.index_scale, a.index_topk, a.window = float(index_scale), int(index_topk), int(window)
        a.q, a.kv = q.data_ptr(), kv.data_ptr()
        a.attn_sink = None if attn_sink is None else attn_sink.data_ptr()
        a.Hq, a.Dqk, a.Dv, a.sm_scale = Hq, Dqk, int(dv), float(sm_scale)
        a.out, a.lse = self.out.data_ptr(), self.lse.data_ptr()
        a.scores = None if self.scores is None else self.scores.data_ptr()
        a.index_list = None if self.index_list is None else self.index_list.data_ptr()
        a.index_flags = DSA_SCORE_RELU if relu else 0
        a.paging = None if paging is None else ctypes.addressof(paging.struct)
        self._args = a
        lib = load_library()
        self.static_scratch = bool(static_scratch)
        self._nws = lib.dsa_decode_step_workspace_size(ctypes.byref(a))
        self._ws = None if self.static_scratch else _workspace(self._nws, dev)
        self.use_graph = bool(graph)
        self._graph = None

    def _launch(self):
        lib = load_library()
        if self.static_scratch:
            _check("dsa_decode_step_static", lib.dsa_decode_step_static(ctypes.byref(self._args), _stream()))
        else:
            _check("dsa_decode_step", lib.dsa_decode_step(ctypes.byref(self._args), _ptr(self._ws), self._nws,
                                                          _stream()))

    def __call__(self):
        if not self.use_graph:
            self._launch()
            return self.out
        if self._graph is None:
            self._launch()  # validates the arguments and loads the kernels outside the capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._launch()
            self._graph = g
        self._graph.replay()
        return self.out


def dsa_decode_step(index_q, index_w, k_cache, **kw):
    """One decode step (score -> top-k + window -> sparse attention).  Returns the DecodeStep
    after running it once: .out [B, 1, Hq, dv] bf16, .lse, .scores, .index_list."""
    step = DecodeStep(index_q, index_w, k_cache, **kw)
    step()
    return step


def dsa_cache_write(k_new, positions, k_cache, *, k_scale=None, rows_per_seq: int = 1, round_scale: bool = False,
                    qdq: bool = False, paging: Optional[Paging] = None, s_max: Optional[int] = None) -> None:
    """Store k_new [T, 128] bf16 into k_cache [T // rows_per_seq, S_max, 128] in place at positions [T] int32.

    An fp8 cache (uint8 / float8_e4m3fn codes, with k_scale [n_seq, S_max] fp32) is written block-quantised;
    a bf16 cache gets the key as is, or quantised and dequantised with ``qdq``.  With ``paging``, k_cache /
    k_scale are page pools [n_pages * page_size, ...] and ``s_max`` the logical slot count."""
    _dev(k_new, "k_new", (torch.bfloat16,))
    _dev(positions, "positions", (torch.int32,))
    _dev(k_cache, "k_cache", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn))
    kd = _key_args(k_cache, k_scale)
    if kd == DSA_KEY_FP8_E4M3 and k_scale is None:
        raise ValueError("an fp8 key cache needs k_scale")
    T, D = k_new.shape
    flags = (DSA_CACHE_ROUND_SCALE if round_scale else 0) | (DSA_CACHE_QDQ if qdq else 0)
    if positions.shape != (T,) or k_cache.shape[-1] != D:
        raise ValueError("shapes: k_new [T, D], positions [T], cache rows of D elements")
    if paging is not None:
        if s_max is None:
            raise ValueError("a paged cache write needs s_max")
        st = load_library().dsa_cache_write_paged(_ptr(k_new), T, int(rows_per_seq), D, _ptr(positions), kd,
                                                  _ptr(k_cache), _ptr(k_scale), ctypes.byref(paging.struct),
                                                  int(s_max), flags, _stream())
        _check("dsa_cache_write_paged", st)
        return
    n_seq, S_max = k_cache.shape[0], k_cache.shape[1]
    if T and n_seq * int(rows_per_seq) != T:
        raise ValueError("k_cache must be [T // rows_per_seq, S_max, D]")
    if k_scale is not None and tuple(k_scale.shape) != (n_seq, S_max):
        raise ValueError("k_scale must be [n_seq, S_max]")
    st = load_library().dsa_cache_write(_ptr(k_new), T, int(rows_per_seq), D, _ptr(positions), kd, _ptr(k_cache),
                                        _ptr(k_scale), S_max, flags, _stream())
    _check("dsa_cache_write", st)
