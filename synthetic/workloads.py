"""The five DSA workloads (shapes and value distributions), at full size or scaled down,
plus prefill-shaped sparse attention (the prefill workload's top-k lists feeding attention).

Every recipe takes its shape parameters as keyword arguments, defaulting to
the full-size workload; tests pass smaller values to get the same structure
at a size the CPU oracle finishes in seconds.  Unstated distributions are
N(0, 1) (query, per-head weights, sinks); "N(0, 0.5)" is read as standard
deviation 0.5.

Tensor ids (keys of the per-tensor Philox streams) are fixed so that every
element is reproducible from (seed, tensor id, leading index).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

from .gen import causal_index_lists, normal, quantize_fp8_blocks, uniform_int

T_INDEX_Q, T_INDEX_W, T_KCACHE, T_POS, T_Q, T_KV, T_SINK, T_LIST = 1, 2, 3, 4, 5, 6, 7, 8

SEED_BASE = 0xD5A00000


@dataclass
class Workload:
    name: str
    seed: int
    # lightning indexer
    index_q: torch.Tensor               # [M, H, D] bf16
    index_w: torch.Tensor               # [M, H] fp32
    k_cache: torch.Tensor               # [M // rows_per_seq, S_max, D] bf16, or uint8 FP8 E4M3 codes
    k_scale: Optional[torch.Tensor]     # [n_seq, S_max] fp32 (FP8 keys only)
    positions: Optional[torch.Tensor]   # [M] int32
    valid_len: int                      # -1: none
    rows_per_seq: int
    index_scale: float
    index_topk: int
    window: int = 0
    # sparse attention (None for indexer-only workloads)
    q: Optional[torch.Tensor] = None    # [B, S, Hq, Dqk] bf16
    kv: Optional[torch.Tensor] = None   # [B, S_kv, Dqk] bf16
    sink: Optional[torch.Tensor] = None  # [Hq] fp32
    sm_scale: float = 0.0
    dv: int = 0
    index_list: Optional[torch.Tensor] = None  # [B, S, K_top] int32 (attention-only workloads)
    meta: dict = field(default_factory=dict)

    @property
    def key_fp8(self) -> bool:
        return self.k_scale is not None

    @property
    def S_max(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def M(self) -> int:
        return int(self.index_q.shape[0])

    def n_valid(self):
        """Attendable slots per row (host-side bookkeeping for reporting only)."""
        S = self.S_max
        if self.positions is not None:
            n = self.positions.to(torch.int64) + 1
        else:
            n = torch.full((self.M,), S, dtype=torch.int64)
        if self.valid_len >= 0:
            n = n.clamp(max=self.valid_len)
        return n.clamp(0, S)


def tiny_decode(seed=SEED_BASE + 1, *, H=4, D=128, S_max=2048, valid_len=1500, topk=64,
                Hq=8, Dqk=192, Dv=128) -> Workload:
    """One query token; 4 indexer heads; 2048 slots, 1500 valid; top-64; attention with
    8 heads over qk 192 (128 + 64 rope) / v 128."""
    return Workload(
        name="tiny_decode", seed=seed,
        index_q=normal(seed, T_INDEX_Q, (1, H, D)),
        index_w=normal(seed, T_INDEX_W, (1, H), dtype=torch.float32),
        k_cache=normal(seed, T_KCACHE, (1, S_max, D)),
        k_scale=None, positions=None, valid_len=valid_len, rows_per_seq=1,
        index_scale=D ** -0.5, index_topk=topk, window=0,
        q=normal(seed, T_Q, (1, 1, Hq, Dqk)),
        kv=normal(seed, T_KV, (1, S_max, Dqk)),
        sink=normal(seed, T_SINK, (Hq,), dtype=torch.float32),
        sm_scale=Dqk ** -0.5, dv=Dv)


def batched_decode(seed=SEED_BASE + 2, *, M=16, H=64, D=128, S_max=32768, pos_lo=4096, topk=1024) -> Workload:
    """16 decode tokens (one per sequence); 64 heads; bf16 cache [16, 32768, 128];
    positions uniform in [4096, 32767], causal valid length position + 1; top-1024."""
    return Workload(
        name="batched_decode", seed=seed,
        index_q=normal(seed, T_INDEX_Q, (M, H, D)),
        index_w=normal(seed, T_INDEX_W, (M, H), dtype=torch.float32),
        k_cache=normal(seed, T_KCACHE, (M, S_max, D)),
        k_scale=None, positions=uniform_int(seed, T_POS, M, pos_lo, S_max - 1), valid_len=-1,
        rows_per_seq=1, index_scale=D ** -0.5, index_topk=topk)


def prefill(seed=SEED_BASE + 3, *, S=8192, H=64, D=128, topk=2048) -> Workload:
    """One sequence of S query tokens scored causally against S keys; 64 heads; top-2048."""
    return Workload(
        name="prefill", seed=seed,
        index_q=normal(seed, T_INDEX_Q, (S, H, D)),
        index_w=normal(seed, T_INDEX_W, (S, H), dtype=torch.float32),
        k_cache=normal(seed, T_KCACHE, (1, S, D)),
        k_scale=None, positions=torch.arange(S, dtype=torch.int32), valid_len=-1,
        rows_per_seq=S, index_scale=D ** -0.5, index_topk=topk)


def fp8_long_decode(seed=SEED_BASE + 4, *, M=4, H=64, D=128, S_max=131072, vl_lo=65536, topk=2048) -> Workload:
    """4 sequences with 131072-slot FP8 E4M3 key caches (one fp32 scale per 128-element
    block = per slot, amax / 448); valid length uniform in [65536, 131072]; top-2048."""
    keys = normal(seed, T_KCACHE, (M, S_max, D), dtype=torch.float32)
    codes, scales = quantize_fp8_blocks(keys)
    del keys
    vl = uniform_int(seed, T_POS, M, vl_lo, S_max)
    return Workload(
        name="fp8_long_decode", seed=seed,
        index_q=normal(seed, T_INDEX_Q, (M, H, D)),
        index_w=normal(seed, T_INDEX_W, (M, H), dtype=torch.float32),
        k_cache=codes, k_scale=scales, positions=(vl - 1).to(torch.int32), valid_len=-1,
        rows_per_seq=1, index_scale=D ** -0.5, index_topk=topk)


def full_decode_step(seed=SEED_BASE + 5, *, B=64, H=64, D=128, S_max=65536, topk=1024, window=128,
                     Hq=128, Dqk=576, Dv=512, kv_sigma=0.5, position=None) -> Workload:
    """Batch of 64 sequences with 65536 cached slots each.  Indexer: 64 heads, top-1024.
    A 128-position sliding window is always selected.  Attention: 128 query heads,
    qk 576 (512 latent + 64 rope), v 512, KV bf16 N(0, 0.5), per-head sink."""
    pos = S_max - 1 if position is None else position
    return Workload(
        name="full_decode_step", seed=seed,
        index_q=normal(seed, T_INDEX_Q, (B, H, D)),
        index_w=normal(seed, T_INDEX_W, (B, H), dtype=torch.float32),
        k_cache=normal(seed, T_KCACHE, (B, S_max, D)),
        k_scale=None, positions=torch.full((B,), pos, dtype=torch.int32), valid_len=-1,
        rows_per_seq=1, index_scale=D ** -0.5, index_topk=topk, window=window,
        q=normal(seed, T_Q, (B, 1, Hq, Dqk)),
        kv=normal(seed, T_KV, (B, S_max, Dqk), sigma=kv_sigma),
        sink=normal(seed, T_SINK, (Hq,), dtype=torch.float32),
        sm_scale=Dqk ** -0.5, dv=Dv)


def prefill_attn(seed=SEED_BASE + 6, *, S=8192, topk=2048, Hq=128, Dqk=576, Dv=512, kv_sigma=0.5) -> Workload:
    """Prefill-shaped sparse attention: one sequence of S = 8192 query tokens, each attending to
    its own causal top-2048 list (min(2048, i + 1) distinct slots of [0, i], -1 padded), with the
    attention of the full decode step (128 heads, qk 576 / v 512, KV N(0, 0.5), per-head sink).
    Attention only: the indexer fields are None."""
    return Workload(
        name="prefill_attn", seed=seed,
        index_q=None, index_w=None, k_cache=None, k_scale=None, positions=None, valid_len=-1,
        rows_per_seq=S, index_scale=0.0, index_topk=topk,
        q=normal(seed, T_Q, (1, S, Hq, Dqk)),
        kv=normal(seed, T_KV, (1, S, Dqk), sigma=kv_sigma),
        sink=normal(seed, T_SINK, (Hq,), dtype=torch.float32),
        sm_scale=Dqk ** -0.5, dv=Dv,
        index_list=causal_index_lists(seed, T_LIST, S, topk).view(1, S, topk))


WORKLOADS = {
    "tiny_decode": tiny_decode,
    "batched_decode": batched_decode,
    "prefill": prefill,
    "fp8_long_decode": fp8_long_decode,
    "full_decode_step": full_decode_step,
    "prefill_attn": prefill_attn,
}


def make_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)


__all__ = ["Workload", "WORKLOADS", "make_workload"]
