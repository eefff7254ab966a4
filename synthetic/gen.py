"""Counter-based seeded draws (numpy Philox-4x64) and storage casts.

Each (seed, tensor id, leading index) triple keys its own Philox stream, so
chunks are generated independently and in parallel, and one chunk can be
regenerated without the rest.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(seed: int, tensor_id: int, chunk: int) -> np.random.Generator:
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, ((tensor_id & 0xFFFFFFFF) << 32) | (chunk & 0xFFFFFFFF)],
                   dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _chunk_normal(seed, tensor_id, chunk, shape, mean, sigma):
    g = _stream(seed, tensor_id, chunk)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def normal(seed: int, tensor_id: int, shape, *, sigma: float = 1.0, mean: float = 0.0,
           dtype: torch.dtype = torch.bfloat16, chunks=None) -> torch.Tensor:
    """N(mean, sigma^2) draws of `shape`, cast to `dtype` (bf16 by RNE), as a CPU tensor.

    The leading axis is the chunk axis: slice i is drawn from stream
    (seed, tensor_id, i).  `chunks` optionally restricts generation to the given
    leading indices (the result then has len(chunks) leading entries).
    """
    shape = tuple(int(s) for s in shape)
    lead = list(range(shape[0])) if chunks is None else [int(c) for c in chunks]
    inner = shape[1:]
    out = torch.empty((len(lead),) + inner, dtype=dtype)

    def work(pos_chunk):
        pos, c = pos_chunk
        x = _chunk_normal(seed, tensor_id, c, inner, mean, sigma)
        out[pos].copy_(torch.from_numpy(x).to(dtype))

    items = list(enumerate(lead))
    if len(items) > 1 and np.prod(inner, dtype=np.int64) >= (1 << 16):
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, items))
    else:
        for it in items:
            work(it)
    return out


def uniform_int(seed: int, tensor_id: int, n: int, lo: int, hi: int) -> torch.Tensor:
    """n integers uniform on [lo, hi] inclusive, int32 CPU tensor."""
    g = _stream(seed, tensor_id, 0)
    return torch.from_numpy(g.integers(lo, hi, size=n, endpoint=True, dtype=np.int64).astype(np.int32))


def causal_index_lists(seed: int, tensor_id: int, S: int, k: int, *, rows=None) -> torch.Tensor:
    """Per-query index lists shaped like a causal top-k: row i holds min(k, i + 1)
    distinct slots drawn uniformly from [0, i] (all of them when i < k), in random
    order, then -1 padding.  int32 [len(rows), k]; row i is drawn from stream
    (seed, tensor_id, i)."""
    rows = list(range(S)) if rows is None else [int(r) for r in rows]
    out = np.full((len(rows), k), -1, dtype=np.int32)

    def work(j):
        i = rows[j]
        g = _stream(seed, tensor_id, i)
        n = min(k, i + 1)
        out[j, :n] = g.permutation(i + 1)[:n] if i + 1 <= 4 * k else g.choice(i + 1, size=n, replace=False)

    if len(rows) > 64:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(len(rows))))
    else:
        for j in range(len(rows)):
            work(j)
    return torch.from_numpy(out)


def page_table(seed: int, tensor_id: int, n_seq: int, max_pages: int, n_pages: int) -> torch.Tensor:
    """Block table of a paged cache: every (sequence, page-of-slots) pair gets a distinct pool page,
    drawn as a random permutation of the n_pages pool pages (n_pages >= n_seq * max_pages; the rest stay
    unused).  int32 [n_seq, max_pages]."""
    assert n_pages >= n_seq * max_pages
    perm = _stream(seed, tensor_id, 0).permutation(n_pages)[: n_seq * max_pages]
    return torch.from_numpy(perm.astype(np.int32).reshape(n_seq, max_pages))


def scatter_pages(x: torch.Tensor, table: torch.Tensor, page_size: int, n_pages: int, fill: torch.Tensor):
    """Storage layout only: the pool [n_pages * page_size, ...] holding x [n_seq, n_slots, ...] page by
    page at the pages the table names; rows no slot maps to are taken from `fill` (same shape as the pool),
    so a read through a wrong page returns unrelated data."""
    n_seq, n_slots = x.shape[0], x.shape[1]
    pool = fill.clone()
    pv = pool.view((n_pages, page_size) + tuple(x.shape[2:]))
    for r in range(n_seq):
        for p in range((n_slots + page_size - 1) // page_size):
            lo, hi = p * page_size, min(n_slots, (p + 1) * page_size)
            pv[int(table[r, p]), : hi - lo] = x[r, lo:hi]
    return pool


def quantize_fp8_blocks(x: torch.Tensor):
    """Store x [..., D] as OCP FP8 E4M3 codes with one fp32 scale per last-axis block.

    Recipe of the DeepSeek-V4 FP8 block quantiser (kwkr.cn article on the
    DeepSeek-V4-Pro-0813-nvfp4-DSpark inference/kernel.py, FP8 block
    quantisation section): scale = amax / 448 per block, data = x / scale
    rounded to the nearest E4M3 value (ties to even) within +-448.  An all-zero
    block gets scale 1.  Returns (codes uint8 [..., D], scales float32 [...]).
    """
    xf = x.to(torch.float32)
    amax = xf.abs().amax(dim=-1)
    scale = amax / 448.0
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    y = (xf / scale.unsqueeze(-1)).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.to(torch.float32).contiguous()
