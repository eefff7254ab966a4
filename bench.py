#!/usr/bin/env python3
"""Benchmark of the DSA decode hot path on one MI355X.

A step is one DSA decode step over a batch: lightning-indexer score of every
cached key slot -> top-k -> index list (top-k plus the always-selected
window) -> top-k sparse attention with sink (dsa_decode_step).  The default
workload is the full decode step: 64 sequences x 65536 cached slots, indexer
64 heads x 128, top-1024, window 128, attention 128 heads, qk 576 / v 512.
Inputs are seeded synthetic tensors, resident in HBM before timing starts.

Prints ONE JSON line with the step throughput (attendable key slots scored
per second through the whole step), per-kernel HIP-event timings, the
roofline of the dominant kernel and the CPU oracle timed on a bounded sample
of the same workload (which also re-checks parity on the timed buffers).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache
METRIC = "DSA decode: indexer key-slots/s + sparse-attn tokens/s; % of HBM peak"
PMC_FILE = os.path.join(ROOT, "profiles", "score_decode_full_decode_step.pmc.json")
KERNEL_SOURCES = {"score_decode": "score_decode.hip", "score_decode_relu": "score_decode_heads.hip", "topk": "topk.hip",
                  "sparse_attn": "sparse_attn.hip", "cache_write": "cache_write.hip"}


def kernel_source_sha(name: str) -> str:
    p = os.path.join(ROOT, "sparse_attention_amd", "csrc", KERNEL_SOURCES[name])
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_decode_step",
                    choices=["full_decode_step", "tiny_decode", "batched_decode", "fp8_long_decode", "prefill",
                             "cache_write", "prefill_attn"])
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--configs", choices=["on", "off"], default="on",
                    help="full_decode_step: also measure the other four configurations (scorer and top-k legs "
                         "of the batched and long fp8 decode indexers and of the prefill scorer, the tiny step)")
    ap.add_argument("--indexer-relu", action="store_true",
                    help="indexer activation max(0, .) per head (per-head MFMA scorer) instead of the identity")
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE",
                    help="decode workloads: keep the key and KV caches in page pools of PAGE slots per page "
                         "(a seeded random page order), read through a block table")
    ap.add_argument("--cpu-sample", type=int, default=64, help="sequences in the oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat oracle passes over the sample until this much time has been spent")
    ap.add_argument("--rotate", type=int, default=0, metavar="R",
                    help="indexer-only workloads: cycle over R copies of the inputs at distinct addresses "
                         "(default: enough copies for twice the 256 MB Infinity Cache, at least 4, when one "
                         "set is smaller than that)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (scale reference for PMC byte counters)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def copy_calibration(torch, dev):
    """Three plain 1 GiB device copies: their PMC byte counters give each counter's scale on this part."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB device copies")
    del src, dst


def event_time_ms(torch, fn, iters):
    """Average duration of fn() over iters launches, HIP events on the current stream."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def graph_time_ms(torch, fn, reps, replays=3, outputs=()):
    """Device time per fn() call: `reps` calls captured in one HIP graph and replayed `replays` times
    between two events, so no host-side launch cost is inside the measurement.  fn must neither allocate
    nor synchronise, and a call sequence of `reps` calls must end where it started (rotations cycle
    completely).  The tensors in `outputs` must hold the same bytes after the replays as after `reps`
    eager calls (every kernel here is deterministic), which checks the captured work."""
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ms = event_time_ms(torch, g.replay, replays) / reps
    for a, b in zip(ref, outputs):
        if not torch.equal(a.view(torch.uint8), b.contiguous().view(torch.uint8)):
            raise RuntimeError("a graph replay gave other results than the eager call")
    del g
    return ms


def rotation_count(args, set_bytes):
    """Copies of the inputs and outputs to cycle over so that each timed call streams from HBM: enough
    for twice the 256 MB Infinity Cache and at least 4 when one set is smaller than that."""
    if args.rotate > 0:
        return args.rotate
    return max(4, -(-2 * MALL_BYTES // set_bytes)) if set_bytes < 2 * MALL_BYTES else 1


def host_threads():
    import oracle

    return oracle.default_threads()


def upload(torch, w, dev):
    c = lambda t: None if t is None else t.contiguous().to(dev)  # noqa: E731
    return c(w.index_q), c(w.index_w), c(w.k_cache), c(w.k_scale), c(w.positions)


def score_bytes_of(w, nv):
    B, H, D = w.index_q.shape
    per_slot = D * (1 if w.key_fp8 else 2) + (4 if w.key_fp8 else 0)
    return int(nv.sum()) * per_slot + B * w.S_max * 4 + B * H * D * 2 + B * H * 4


def indexer_legs(args, torch, dsa, w, dev, relu=False, paging=None, s_max=None):
    """Scorer and top-k of a decode indexer workload, each timed from replayed HIP graphs over rotated
    input sets with every output and workspace allocated beforehand.  Returns the timings and the first
    set's scores and top-k rows."""
    B = w.M
    S_max = w.S_max
    k = w.index_topk
    pkw = {"paging": paging, "s_max": s_max} if paging is not None else {}
    base = upload(torch, w, dev)
    if paging is not None:
        base = (base[0], base[1], args._pool_k, args._pool_ks, base[4])
    scores = torch.empty((B, S_max), dtype=torch.float32, device=dev)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    nws = dsa.topk_workspace_bytes(B, S_max, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    set_bytes = sum(t.numel() * t.element_size() for t in base + (scores, idx) if t is not None)
    n_rot = 1 if paging is not None else rotation_count(args, set_bytes)
    sets = [base + (scores, idx)]
    for _ in range(n_rot - 1):
        sets.append(tuple(None if t is None else t.clone() for t in sets[0]))
    torch.cuda.synchronize()
    rot = [0]

    def nxt():
        i = rot[0]
        rot[0] = (i + 1) % n_rot
        return sets[i]

    def score_once():
        q_, w_, k_, ks_, pos_, sc_, _ = nxt()
        dsa.dsa_index_score(q_, w_, k_, scale=w.index_scale, k_scale=ks_, positions=pos_, valid_len=w.valid_len,
                            relu=relu, out=sc_, **pkw)

    def topk_once():
        _, _, _, _, pos_, sc_, id_ = nxt()
        dsa.dsa_topk(sc_, k, positions=pos_, valid_len=w.valid_len, out=id_, workspace=ws)

    reps = max(args.steps, n_rot)
    reps -= reps % n_rot
    ms_score = graph_time_ms(torch, score_once, reps, outputs=[s[5] for s in sets])
    rot[0] = 0
    ms_topk = graph_time_ms(torch, topk_once, reps, outputs=[s[6] for s in sets])
    return ms_score, ms_topk, n_rot, scores, idx


def indexer_entry(w, nv, ms_score, ms_topk, n_rot):
    sb = score_bytes_of(w, nv)
    n_slots = int(nv.sum())
    tb = n_slots * 4 + w.M * w.index_topk * 4
    return {"score_us": ms_score * 1e3, "score_GB/s": sb / ms_score / 1e6,
            "score_hbm_frac": sb / ms_score / 1e6 / HBM_PEAK_GBS, "score_bytes": sb,
            "key_slots_per_s": n_slots / ms_score * 1e3, "topk_us": ms_topk * 1e3, "topk_bytes": tb,
            "input_sets": n_rot}


def config_indexer(args, torch, dsa, synthetic, dev, name, number):
    """Configs 2 and 4 (decode indexer only): scorer and top-k legs with rotation, parity on sampled rows."""
    import oracle
    from parity import check_scores, check_topk_own_scores, n_valid_rows

    w = synthetic.make_workload(name)
    nv = w.n_valid().numpy()
    ms_s, ms_t, n_rot, scores, idx = indexer_legs(args, torch, dsa, w, dev)
    e = {"config": number, **indexer_entry(w, nv, ms_s, ms_t, n_rot)}
    rows = np.array([0, w.M - 1])
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache[rows],
                             k_scale=None if w.k_scale is None else w.k_scale[rows], scale=w.index_scale,
                             positions=w.positions[rows], valid_len=w.valid_len)
    check_scores(scores.cpu().numpy()[rows], ref, nv[rows], oracle.mask_bound())
    check_topk_own_scores(idx.cpu().numpy()[rows], ref, nv[rows], w.index_topk)
    e["parity"] = "ok (rows %s)" % rows.tolist()
    log("config %d %s: score %.1f us (%.1f%% HBM), top-k %.1f us, %d input sets" % (
        number, name, e["score_us"], 100 * e["score_hbm_frac"], e["topk_us"], n_rot))
    return e


def config_prefill(args, torch, dsa, synthetic, dev):
    """Config 3: the prefill scorer (identity: heads folded, HBM-bound on the score writes; ReLU: per-head
    MFMA) and the prefill top-k, with rotation, parity on sampled rows."""
    import oracle
    from parity import check_scores, check_topk_own_scores

    w = synthetic.make_workload("prefill")
    S, H, D = w.index_q.shape
    gq, gw, gk, _, gpos = upload(torch, w, dev)
    scores = torch.empty((S, S), dtype=torch.float32, device=dev)
    idx = torch.empty((S, w.index_topk), dtype=torch.int32, device=dev)
    set_bytes = sum(t.numel() * t.element_size() for t in (gq, gw, gk, gpos, scores, idx))
    n_rot = rotation_count(args, set_bytes)
    sets = [(gq, gw, gk, gpos, scores, idx)] + [
        tuple(t.clone() for t in (gq, gw, gk, gpos, scores, idx)) for _ in range(n_rot - 1)]
    torch.cuda.synchronize()
    rot = [0]

    def nxt():
        i = rot[0]
        rot[0] = (i + 1) % n_rot
        return sets[i]

    def score(relu):
        def f():
            q_, w_, k_, p_, sc_, _ = nxt()
            dsa.dsa_index_score(q_, w_, k_, scale=w.index_scale, positions=p_, rows_per_seq=S, relu=relu, out=sc_)
        return f

    def topk_once():
        _, _, _, p_, sc_, id_ = nxt()
        dsa.dsa_topk(sc_, w.index_topk, positions=p_, out=id_)

    reps = n_rot * max(1, args.steps // (2 * n_rot))
    pairs = S * (S + 1) // 2
    flops = 2.0 * H * D * pairs
    nbytes = S * S * 4 + S * H * D * 2 + S * H * 4 + S * D * 2
    ms_relu = graph_time_ms(torch, score(True), reps, outputs=[s[4] for s in sets])
    rot[0] = 0
    ms_fold = graph_time_ms(torch, score(False), reps, outputs=[s[4] for s in sets])
    rot[0] = 0
    ms_topk = graph_time_ms(torch, topk_once, reps, outputs=[s[5] for s in sets])
    rows = np.array([0, 31, 2047, 4096, 6001, S - 1])
    sc = scores[torch.from_numpy(rows).to(dev)].cpu().numpy()
    ref = oracle.index_score(w.index_q[rows], w.index_w[rows], w.k_cache, scale=w.index_scale,
                             positions=w.positions[rows], rows_per_seq=len(rows))
    check_scores(sc, ref, rows + 1, oracle.mask_bound())
    check_topk_own_scores(idx.cpu().numpy()[rows], ref, rows + 1, w.index_topk)
    e = {"config": 3, "score_fold_us": ms_fold * 1e3, "score_fold_GB/s": nbytes / ms_fold / 1e6,
         "score_fold_hbm_frac": nbytes / ms_fold / 1e6 / HBM_PEAK_GBS, "score_fold_bytes": nbytes,
         "score_relu_us": ms_relu * 1e3, "score_relu_TFLOP/s": flops / ms_relu / 1e9,
         "score_relu_mfma_frac": flops / ms_relu / 1e9 / MFMA_BF16_PEAK_TFLOPS, "per_head_flops": flops,
         "topk_us": ms_topk * 1e3, "input_sets": n_rot, "parity": "ok (identity scores, rows %s)" % rows.tolist()}
    log("config 3 prefill: fold score %.1f us (%.1f%% HBM), ReLU score %.1f us (%.1f%% MFMA), top-k %.1f us" % (
        e["score_fold_us"], 100 * e["score_fold_hbm_frac"], e["score_relu_us"], 100 * e["score_relu_mfma_frac"],
        e["topk_us"]))
    return e


def config_tiny(args, torch, dsa, synthetic, dev):
    """Config 1: the tiny decode step, timed from a replayed graph, checked whole against the oracle."""
    import oracle
    from parity import check_attn, check_index_list, check_scores, n_valid_rows

    w = synthetic.make_workload("tiny_decode")
    gq, gw, gk, _, _ = upload(torch, w, dev)
    c = lambda t: t.contiguous().to(dev)  # noqa: E731
    step = dsa.DecodeStep(gq, gw, gk, valid_len=w.valid_len, index_scale=w.index_scale, index_topk=w.index_topk,
                          window=w.window, q=c(w.q), kv=c(w.kv), attn_sink=c(w.sink), sm_scale=w.sm_scale, dv=w.dv)
    ms = graph_time_ms(torch, step, 50, outputs=[step.out, step.index_list])
    nv = n_valid_rows(None, w.valid_len, 1, w.S_max)
    ref_sc = oracle.index_score(w.index_q, w.index_w, w.k_cache, scale=w.index_scale, valid_len=w.valid_len)
    check_scores(step.scores.cpu().numpy(), ref_sc, nv, oracle.mask_bound())
    ref_top = oracle.topk(ref_sc, w.index_topk, valid_len=w.valid_len)
    ref_list = oracle.assemble(ref_top, s_max=w.S_max, window=w.window, valid_len=w.valid_len)
    check_index_list(step.index_list.cpu().numpy(), ref_list, ref_sc, nv, w.index_topk, w.window)
    ref_out, _ = oracle.sparse_attn(w.q, w.kv, w.sink, step.index_list.cpu().numpy()[:, None, :],
                                    sm_scale=w.sm_scale, dv=w.dv)
    err, rel = check_attn(step.out.float().cpu().numpy(), ref_out)
    log("config 1 tiny_decode: step %.1f us" % (ms * 1e3))
    return {"config": 1, "step_us": ms * 1e3, "parity": "ok (whole step; attention max abs %.2g, rel-L2 %.2g)" % (
        err, rel)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this DSA hot path is measured on exactly one GPU; --gpus %d (WORLD_SIZE %d) is not "
              "supported. Sharding across GPUs is a design note only." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_amd as dsa
    import synthetic

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    dsa.load_library()
    dev = torch.device("cuda:0")
    t0 = time.time()
    if args.copy_calibration and args.workload in ("prefill", "cache_write", "prefill_attn"):
        copy_calibration(torch, dev)  # (the decode workloads run it after their timings)
    if args.workload == "prefill":
        return bench_prefill(args, torch, dsa, synthetic, dev)
    if args.workload == "cache_write":
        return bench_cache_write(args, torch, dsa, synthetic, dev)
    if args.workload == "prefill_attn":
        return bench_prefill_attn(args, torch, dsa, synthetic, dev)
    w = synthetic.make_workload(args.workload)
    log("generated %s in %.1fs" % (args.workload, time.time() - t0))
    gq, gw, gk, gks, gpos = upload(torch, w, dev)
    has_attn = w.q is not None
    if has_attn:
        c = lambda t: t.contiguous().to(dev)  # noqa: E731
        gaq, gkv, gsink = c(w.q), c(w.kv), c(w.sink)
    torch.cuda.synchronize()
    log("inputs resident on %s" % torch.cuda.get_device_name(0))

    B, H, D = w.index_q.shape
    S_max = w.S_max
    nv = w.n_valid().numpy()
    n_slots = int(nv.sum())
    k = w.index_topk
    K_top = k + w.window

    paging = None
    pkw = {}
    if args.paged:
        # page pools in a seeded random page order; the contiguous copies are dropped
        P = args.paged
        max_pages = (S_max + P - 1) // P
        n_pages = B * max_pages
        table = synthetic.page_table(w.seed, 99, B, max_pages, n_pages)
        dst = table.flatten().long().to(dev)

        def to_pool(x):
            if x is None:
                return None
            pad = max_pages * P - S_max
            if pad:
                x = torch.nn.functional.pad(x.view(B, S_max, -1), (0, 0, 0, pad)).view((B, max_pages * P) +
                                                                                     tuple(x.shape[2:]))
            pool = torch.empty((n_pages * P,) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
            pool.view((n_pages, P) + tuple(x.shape[2:]))[dst] = x.reshape((B * max_pages, P) + tuple(x.shape[2:]))
            return pool

        gk, gks = to_pool(gk), to_pool(gks)
        args._pool_k, args._pool_ks = gk, gks
        if has_attn:
            gkv = to_pool(gkv)
        torch.cuda.synchronize()
        paging = dsa.Paging(table.to(dev), P, n_pages)
        pkw = {"paging": paging}
        log("page pools: %d pages of %d slots" % (n_pages, P))

    # ---- the step (the headline number): eager calls between two events
    if has_attn:
        step = dsa.DecodeStep(gq, gw, gk, k_scale=gks, positions=gpos, valid_len=w.valid_len,
                              index_scale=w.index_scale, index_topk=k, window=w.window, q=gaq, kv=gkv,
                              attn_sink=gsink, sm_scale=w.sm_scale, dv=w.dv, relu=args.indexer_relu,
                              s_max=S_max if paging else None, **pkw)
        run_step = step
        n_rot = 1
    else:
        scores_buf = torch.empty((B, S_max), dtype=torch.float32, device=dev)
        idx_buf = torch.empty((B, k), dtype=torch.int32, device=dev)
        nws = dsa.topk_workspace_bytes(B, S_max, k)
        ws_buf = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        set_bytes = sum(t.numel() * t.element_size() for t in (gq, gw, gk, gks, gpos, scores_buf) if t is not None)
        n_rot = 1 if paging else rotation_count(args, set_bytes)
        sets = [(gq, gw, gk, gks, gpos, scores_buf)]
        for _ in range(n_rot - 1):
            sets.append(tuple(None if t is None else t.clone() for t in sets[0]))
        torch.cuda.synchronize()
        if n_rot > 1:
            log("rotating over %d input sets of %.1f MB (%.0f MB in all)" % (n_rot, set_bytes / 1e6,
                                                                          n_rot * set_bytes / 1e6))
        rot = [0]

        def run_step():
            i = rot[0]
            rot[0] = (i + 1) % n_rot
            q_, w_, k_, ks_, pos_, sc_ = sets[i]
            dsa.dsa_index_score(q_, w_, k_, scale=w.index_scale, k_scale=ks_, positions=pos_,
                                valid_len=w.valid_len, relu=args.indexer_relu, out=sc_,
                                s_max=S_max if paging else None, **pkw)
            dsa.dsa_topk(sc_, k, positions=pos_, valid_len=w.valid_len, out=idx_buf, workspace=ws_buf)

    # Untimed settling before the W warm-up steps: the first ~0.1 s of steps after the inputs are generated run
    # slower (clocks still ramping, first touches of the page tables of the multi-GB caches); a short W would
    # otherwise leave that in the timed steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.1:
        for _ in range(10):
            run_step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_step = event_time_ms(torch, run_step, args.steps)
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    log("step %.3f ms (host wall %.3f ms/step)" % (ms_step, wall_ms))

    # ---- per-kernel legs: replayed HIP graphs, every output and workspace allocated beforehand
    ms_score, ms_topk, n_rot_legs, scores_leg, _ = indexer_legs(
        args, torch, dsa, w, dev, relu=args.indexer_relu, paging=paging, s_max=S_max if paging else None)
    score_name = "score_decode_relu" if args.indexer_relu else "score_decode"
    e = indexer_entry(w, nv, ms_score, ms_topk, n_rot_legs)
    kern = {score_name: {"us": e["score_us"], "bytes": e["score_bytes"], "GB/s": e["score_GB/s"],
                         "hbm_frac": e["score_hbm_frac"], "key_slots_per_s": e["key_slots_per_s"]},
            "topk": {"us": e["topk_us"], "bytes": e["topk_bytes"], "GB/s": e["topk_bytes"] / ms_topk / 1e6,
                     "note": "standalone dsa_topk, including its header-clear launch (in the step the scorer "
                             "clears the header)"}}
    step_bytes = e["score_bytes"] + e["topk_bytes"]
    if has_attn:
        lst = step.index_list.view(B, 1, K_top)
        n_entries = int((step.index_list >= 0).sum().item())
        Hq, Dqk, Dv = w.q.shape[2], w.q.shape[3], w.dv
        attn_bytes = n_entries * Dqk * 2 + B * Hq * Dqk * 2 + B * Hq * Dv * 2 + B * K_top * 4
        attn_flops = 2.0 * Hq * n_entries * (Dqk + Dv)
        attn_out = torch.empty((B, 1, Hq, Dv), dtype=torch.bfloat16, device=dev)
        nws_a = dsa.sparse_attn_workspace_bytes(B, 1, Hq, Dv, K_top)
        ws_a = torch.empty(max(nws_a, 1), dtype=torch.uint8, device=dev)
        ms_attn = graph_time_ms(torch, lambda: dsa.dsa_sparse_attn(
            gaq, gkv, gsink, lst, sm_scale=w.sm_scale, dv=Dv, out=attn_out, workspace=ws_a,
            s_kv=S_max if paging else None, **pkw), args.steps, outputs=[attn_out])
        if not torch.equal(attn_out, step.out):
            raise RuntimeError("the attention leg differs from the step's attention on the same list")
        kern["sparse_attn"] = {"us": ms_attn * 1e3, "bytes": attn_bytes, "flops": attn_flops,
                               "GB/s": attn_bytes / ms_attn / 1e6,
                               "hbm_frac": attn_bytes / ms_attn / 1e6 / HBM_PEAK_GBS,
                               "mfma_frac": attn_flops / ms_attn / 1e9 / MFMA_BF16_PEAK_TFLOPS,
                               "tokens_per_s": B / ms_attn * 1e3,
                               "kv_entries_per_s": n_entries / ms_attn * 1e3}
        step_bytes += attn_bytes
        ms_step_graph = graph_time_ms(torch, step, max(4, args.steps // 2), outputs=[step.out, step.index_list])
        log("step from a replayed graph %.3f ms" % ms_step_graph)
    for name, v in kern.items():
        log("%-12s %9.2f us  %8.1f GB/s" % (name, v["us"], v["GB/s"]))

    if args.copy_calibration:
        copy_calibration(torch, dev)

    # ---- dominant kernel roofline (HBM-bound streaming scorer)
    dom = max(kern, key=lambda n: kern[n]["us"])
    traffic = None
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as f:
            pmc = json.load(f)
        if pmc.get("kernel") == dom and pmc.get("source_sha") == kernel_source_sha(dom) and \
                pmc.get("workload") == args.workload and not args.paged and not args.indexer_relu:
            traffic = pmc.get("hbm_bytes_per_launch")
    if dom == "sparse_attn":
        roof = {"bound": "mfma", "achieved": attn_flops / ms_attn / 1e9, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = dom

    # ---- the other configurations, measured in this run (default workload only)
    configs = None
    if args.workload == "full_decode_step" and args.configs == "on" and not args.paged and not args.indexer_relu:
        configs = {"full_decode_step": {
            "config": 5, "step_us": ms_step * 1e3, "step_graph_us": ms_step_graph * 1e3,
            "step_hbm_frac": step_bytes / ms_step / 1e6 / HBM_PEAK_GBS, "score_us": kern[score_name]["us"],
            "score_hbm_frac": kern[score_name]["hbm_frac"], "topk_us": kern["topk"]["us"],
            "attn_us": kern["sparse_attn"]["us"], "attn_hbm_frac": kern["sparse_attn"]["hbm_frac"],
            "attn_mfma_frac": kern["sparse_attn"]["mfma_frac"]}}
        configs["tiny_decode"] = config_tiny(args, torch, dsa, synthetic, dev)
        configs["batched_decode"] = config_indexer(args, torch, dsa, synthetic, dev, "batched_decode", 2)
        torch.cuda.empty_cache()
        configs["prefill"] = config_prefill(args, torch, dsa, synthetic, dev)
        torch.cuda.empty_cache()
        configs["fp8_long_decode"] = config_indexer(args, torch, dsa, synthetic, dev, "fp8_long_decode", 4)
        torch.cuda.empty_cache()

    # ---- CPU oracle on a bounded sample of the same workload (+ parity on the timed buffers)
    cpu = None
    parity = None
    if args.cpu_baseline == "on":
        scores_t = step.scores if has_attn else scores_leg
        cpu, parity = cpu_baseline(args, w, step if has_attn else None, scores_t, nv, torch)
        if args.workload == "full_decode_step" and not args.paged and not args.indexer_relu:
            cpu["single_thread"] = single_thread_rates(args, synthetic)

    rec = {
        "metric": METRIC,
        "value": n_slots / ms_step * 1e3,
        "unit": "key-slots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "cache_slots": S_max, "attendable_slots": n_slots,
                   "index_heads": H, "head_dim": D, "key_dtype": "fp8_e4m3" if w.key_fp8 else "bf16",
                   "index_topk": k, "window": w.window,
                   "indexer_activation": "relu" if args.indexer_relu else "identity",
                   "kv_layout": ("paged, %d-slot pages" % args.paged) if args.paged else "contiguous",
                   "input_sets": n_rot,
                   **({"attn_heads": int(w.q.shape[2]), "dqk": int(w.q.shape[3]), "dv": w.dv} if has_attn else {}),
                   "parallelism": "single-gpu"},
        "decode_tokens_per_s": B / ms_step * 1e3,
        "step_hbm_frac": step_bytes / ms_step / 1e6 / HBM_PEAK_GBS,
        "indexer_key_slots_per_s": kern[score_name]["key_slots_per_s"],
        "sparse_attn_tokens_per_s": kern["sparse_attn"]["tokens_per_s"] if has_attn else None,
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "configs": configs,
    }
    print(json.dumps(rec), flush=True)


def bench_prefill(args, torch, dsa, synthetic, dev):
    """Prefill indexer: 8192 queries scored causally against 8192 keys, then top-2048.  With the identity
    activation the heads fold into one query per row and the kernel is bound by writing the 8192 x 8192
    score matrix (HBM roofline); with --indexer-relu it runs the per-head MFMA contraction (MFMA roofline)."""
    w = synthetic.make_workload("prefill")
    c = lambda t: None if t is None else t.contiguous().to(dev)  # noqa: E731
    gq, gw, gk, gpos = c(w.index_q), c(w.index_w), c(w.k_cache), c(w.positions)
    S, H, D = w.index_q.shape
    relu = args.indexer_relu
    scores = torch.empty((S, S), dtype=torch.float32, device=dev)

    def run_score():
        dsa.dsa_index_score(gq, gw, gk, scale=w.index_scale, positions=gpos, rows_per_seq=S, relu=relu, out=scores)

    for _ in range(args.warmup):
        run_score()
    torch.cuda.synchronize()
    ms = event_time_ms(torch, run_score, args.steps)
    pairs = S * (S + 1) // 2
    flops = 2.0 * H * D * pairs  # the per-head contraction (the folded kernel does 1/H of it)
    run_topk = lambda: dsa.dsa_topk(scores, w.index_topk, positions=gpos)  # noqa: E731
    for _ in range(args.warmup):
        run_topk()
    torch.cuda.synchronize()
    ms_topk = event_time_ms(torch, run_topk, args.steps)
    tflops = flops / ms / 1e9
    nbytes = S * S * 4 + S * H * D * 2 + S * H * 4 + S * D * 2  # scores out, q, w, keys
    gbs = nbytes / ms / 1e6
    if relu:
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "kernel": "score_prefill"}
        log("prefill score (per-head, ReLU) %.1f us: %.1f TFLOP/s (%.1f%% of bf16 MFMA peak); top-k %.1f us" % (
            ms * 1e3, tflops, 100 * tflops / MFMA_BF16_PEAK_TFLOPS, ms_topk * 1e3))
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "traffic": None, "kernel": "score_prefill_fold"}
        log("prefill score (heads folded) %.1f us: %.0f GB/s (%.1f%% of HBM); top-k %.1f us" % (
            ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, ms_topk * 1e3))
    rec = {"metric": METRIC, "value": pairs / ms * 1e3, "unit": "query-key pairs/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prefill", "queries": S, "keys": S, "index_heads": H, "head_dim": D,
                      "index_topk": w.index_topk, "indexer_activation": "relu" if relu else "identity",
                      "parallelism": "single-gpu"},
           "kernels": {("score_prefill" if relu else "score_prefill_fold"):
                       {"us": ms * 1e3, "bytes": nbytes, "GB/s": gbs, "per_head_flops": flops,
                        "per_head_TFLOP/s_equivalent": tflops},
                       "topk": {"us": ms_topk * 1e3}},
           "roofline": roof,
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def bench_prefill_attn(args, torch, dsa, synthetic, dev):
    """Prefill-shaped sparse attention: 8192 query tokens of one sequence, each over its own causal
    top-2048 list, 128 heads, qk 576 / v 512 (MFMA-bound: the 9.4 MB KV stays in cache)."""
    import numpy as np

    t0 = time.time()
    w = synthetic.make_workload("prefill_attn")
    log("generated prefill_attn in %.1fs" % (time.time() - t0))
    gq, gkv, gsink, glist = (t.contiguous().to(dev) for t in (w.q, w.kv, w.sink, w.index_list))
    B, S, Hq, Dqk = w.q.shape
    Dv, K_top = w.dv, w.index_list.shape[2]
    out = torch.empty((B, S, Hq, Dv), dtype=torch.bfloat16, device=dev)
    run = lambda: dsa.dsa_sparse_attn(gq, gkv, gsink, glist, sm_scale=w.sm_scale, dv=Dv, out=out)  # noqa: E731
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ms = event_time_ms(torch, run, args.steps)
    n_entries = int((w.index_list >= 0).sum().item())
    flops = 2.0 * Hq * n_entries * (Dqk + Dv)
    tflops = flops / ms / 1e9
    gathered = n_entries * Dqk * 2 + B * S * Hq * (Dqk + Dv) * 2 + B * S * K_top * 4
    log("prefill sparse attention %.1f us: %.1f TFLOP/s (%.1f%% of bf16 MFMA peak)" % (
        ms * 1e3, tflops, 100 * tflops / MFMA_BF16_PEAK_TFLOPS))
    cpu = None
    if args.cpu_baseline == "on":
        import oracle

        rows = [0, 2047, 2048, S - 1]
        sl = torch.tensor(rows)
        nthr = oracle.default_threads()
        t0 = time.perf_counter()
        ref, _ = oracle.sparse_attn(w.q[:, sl], w.kv, w.sink, w.index_list[:, sl], sm_scale=w.sm_scale, dv=Dv,
                                    nthreads=nthr)
        sec = time.perf_counter() - t0
        err = float(np.abs(out[:, sl.to(dev)].float().cpu().numpy() - ref).max())
        cpu = {"value": len(rows) / sec, "unit": "query tokens/s", "cores": nthr, "kind": "oracle", "seconds": sec,
               "sample": "query tokens %s (all 128 heads each)" % rows, "attention_max_abs_err": err}
    rec = {"metric": METRIC, "value": B * S / ms * 1e3, "unit": "query tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prefill_attn", "queries": S, "index_topk": K_top, "attended_entries": n_entries,
                      "attn_heads": Hq, "dqk": Dqk, "dv": Dv, "parallelism": "single-gpu"},
           "kernels": {"sparse_attn": {"us": ms * 1e3, "flops": flops, "TFLOP/s": tflops,
                                       "bytes": gathered, "GB/s": gathered / ms / 1e6}},
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "kernel": "sparse_attn"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def bench_cache_write(args, torch, dsa, synthetic, dev):
    """Key-cache write with FP8 block quantisation: the whole long-context fp8 cache (4 x 131072 keys of
    128 bf16) quantised in one call, and the decode-shaped write of one new key per sequence (64 sequences
    of 65536 slots)."""
    n_seq, S_max = 4, 131072
    T = n_seq * S_max
    keys = synthetic.normal(41, 0, (T, 128))
    gk = keys.to(dev)
    gpos = torch.arange(S_max, dtype=torch.int32, device=dev).repeat(n_seq)
    kc = torch.empty((n_seq, S_max, 128), dtype=torch.uint8, device=dev)
    ks = torch.empty((n_seq, S_max), dtype=torch.float32, device=dev)
    run = lambda: dsa.dsa_cache_write(gk, gpos, kc, k_scale=ks, rows_per_seq=S_max)  # noqa: E731
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ms = event_time_ms(torch, run, args.steps)
    tok_bytes = 128 * 2 + 4 + 128 + 4  # key read, position read, codes and scale written
    gbs = T * tok_bytes / ms / 1e6
    # decode shape: 64 new keys, one per sequence, into a 64 x 65536-slot fp8 cache
    B, S_dec = 64, 65536
    dk = synthetic.normal(42, 0, (B, 128)).to(dev)
    dpos = torch.full((B,), S_dec - 1, dtype=torch.int32, device=dev)
    dkc = torch.empty((B, S_dec, 128), dtype=torch.uint8, device=dev)
    dks = torch.empty((B, S_dec), dtype=torch.float32, device=dev)
    run_dec = lambda: dsa.dsa_cache_write(dk, dpos, dkc, k_scale=dks)  # noqa: E731
    for _ in range(args.warmup):
        run_dec()
    torch.cuda.synchronize()
    ms_dec_host = event_time_ms(torch, run_dec, args.steps)  # bound by the host-side call at this size
    # the kernel alone: 32 launches captured in a HIP graph, replayed (the write allocates and clears nothing)
    ref_c = dkc[:, S_dec - 1].clone()
    ref_s = dks[:, S_dec - 1].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(32):
            run_dec()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ms_dec = event_time_ms(torch, graph.replay, args.steps) / 32
    if not (torch.equal(dkc[:, S_dec - 1], ref_c) and torch.equal(dks[:, S_dec - 1], ref_s)):
        raise RuntimeError("graph replays of the decode-shaped cache write differ from the eager call")
    log("cache write: %d keys in %.1f us (%.0f GB/s, %.1f%% of HBM); 64 decode keys in %.2f us (%.2f us per host call)" % (
        T, ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, ms_dec * 1e3, ms_dec_host * 1e3))
    cpu = None
    if args.cpu_baseline == "on":
        import oracle

        n_threads = 1  # the oracle's quantiser is a single-threaded loop
        sample = keys[: 1 << 15]
        t0 = time.perf_counter()
        reps = 0
        while True:
            codes, scales = oracle.quantize_fp8_blocks(sample)
            reps += 1
            if time.perf_counter() - t0 >= min(args.cpu_seconds, 5.0):
                break
        sec = time.perf_counter() - t0
        got_c = kc.view(-1, 128)[: sample.shape[0]].cpu().numpy()
        got_s = ks.view(-1)[: sample.shape[0]].cpu().numpy()
        import numpy as np

        cpu = {"value": reps * sample.shape[0] / sec, "unit": "keys/s", "cores": n_threads, "kind": "oracle",
               "seconds": sec, "sample": "%d pass(es) over the first %d of the %d keys" % (reps, sample.shape[0], T),
               "parity": "ok" if np.array_equal(got_c, codes) and np.array_equal(got_s, scales[:, 0])
               else "MISMATCH"}
    rec = {"metric": METRIC, "value": T / ms * 1e3, "unit": "keys/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "cache_write", "sequences": n_seq, "cache_slots": S_max, "keys": T,
                      "head_dim": 128, "key_dtype": "fp8_e4m3", "quant_block": 128, "parallelism": "single-gpu"},
           "kernels": {"cache_write": {"us": ms * 1e3, "bytes": T * tok_bytes, "GB/s": gbs,
                                       "hbm_frac": gbs / HBM_PEAK_GBS},
                       "cache_write_decode64": {"us": ms_dec * 1e3, "us_host_call": ms_dec_host * 1e3,
                                                "bytes": B * tok_bytes}},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "cache_write"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def single_thread_rates(args, synthetic):
    """The oracle on one thread for configs 1, 2 and 4: the whole tiny step, and score + top-k of one
    sequence of the batched and the long fp8 decode, each repeated for about two seconds."""
    import oracle

    out = {}
    budget = min(2.0, args.cpu_seconds)

    def timed(fn):
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget:
                return n, time.perf_counter() - t0

    w = synthetic.make_workload("tiny_decode")
    nv = int(w.n_valid().sum())

    def tiny():
        sc = oracle.index_score(w.index_q, w.index_w, w.k_cache, scale=w.index_scale, valid_len=w.valid_len,
                                nthreads=1)
        top = oracle.topk(sc, w.index_topk, valid_len=w.valid_len, nthreads=1)
        lst = oracle.assemble(top, s_max=w.S_max, window=w.window, valid_len=w.valid_len)
        oracle.sparse_attn(w.q, w.kv, w.sink, lst[:, None, :], sm_scale=w.sm_scale, dv=w.dv, nthreads=1)

    n, sec = timed(tiny)
    out["tiny_decode"] = {"config": 1, "value": n * nv / sec, "unit": "key-slots/s", "steps_per_s": n / sec,
                          "sample": "%d whole step(s): score + full-sort top-k + attention" % n}
    for name, number in (("batched_decode", 2), ("fp8_long_decode", 4)):
        w = synthetic.make_workload(name)
        r = slice(0, 1)
        nv0 = int(w.n_valid()[0])

        def one(w=w, r=r):
            sc = oracle.index_score(w.index_q[r], w.index_w[r], w.k_cache[r],
                                    k_scale=None if w.k_scale is None else w.k_scale[r], scale=w.index_scale,
                                    positions=w.positions[r], valid_len=w.valid_len, nthreads=1)
            oracle.topk(sc, w.index_topk, positions=w.positions[r], valid_len=w.valid_len, nthreads=1)

        n, sec = timed(one)
        out[name] = {"config": number, "value": n * nv0 / sec, "unit": "key-slots/s",
                     "sample": "%d pass(es) of score + full-sort top-k over sequence 0 (%d attendable slots)" % (
                         n, nv0)}
        del w
    for v in out.values():
        v["cores"] = 1
    log("oracle on one thread: " + ", ".join("%s %.3g key-slots/s" % (k, v["value"]) for k, v in out.items()))
    return out


def cpu_baseline(args, w, step, scores_t, nv, torch):
    """Time the oracle (as it stands) on `cpu_sample` sequences of the same workload, and check the
    GPU's outputs for those sequences against it."""
    import oracle

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import check_attn, check_index_list, check_scores, check_topk_own_scores

    ns = min(args.cpu_sample, w.M)
    rows = np.linspace(0, w.M - 1, ns).round().astype(np.int64)
    threads = oracle.default_threads()  # every core in the affinity mask, or OMP_NUM_THREADS if set lower
    whole = ns == w.M  # the sample is the whole batch: no copies
    sub = lambda t: None if t is None else (t if whole else t[rows])  # noqa: E731
    pos = sub(w.positions)
    sub_q, sub_w, sub_k, sub_ks = sub(w.index_q), sub(w.index_w), sub(w.k_cache), sub(w.k_scale)
    sub_aq, sub_kv = (sub(w.q), sub(w.kv)) if step is not None else (None, None)
    def one_pass():
        sc = oracle.index_score(sub_q, sub_w, sub_k, k_scale=sub_ks, scale=w.index_scale,
                                positions=pos, valid_len=w.valid_len, relu=args.indexer_relu, nthreads=threads)
        top = oracle.topk(sc, w.index_topk, positions=pos, valid_len=w.valid_len, nthreads=threads)
        lst = out = None
        if step is not None:
            lst = oracle.assemble(top, s_max=w.S_max, window=w.window, positions=pos, valid_len=w.valid_len)
            out, _ = oracle.sparse_attn(sub_aq, sub_kv, w.sink, lst[:, None, :], sm_scale=w.sm_scale,
                                        dv=w.dv, nthreads=threads)
        return sc, lst, out

    # whole passes over the sample until cpu_seconds have gone by (a steadier rate than one pass)
    t0 = time.perf_counter()
    ref_sc, ref_list, ref_out = one_pass()
    passes = 1
    while time.perf_counter() - t0 < args.cpu_seconds:
        one_pass()
        passes += 1
    secs = time.perf_counter() - t0
    n_slots = int(nv[rows].sum()) * passes
    log("oracle: %d x %d sequences in %.1fs on %d threads" % (passes, ns, secs, threads))
    parity = {}
    check_scores(scores_t[torch.from_numpy(rows).to(scores_t.device)].cpu().numpy(), ref_sc, nv[rows],
                 oracle.mask_bound())
    parity["scores"] = "ok"
    if step is None:
        # the indexer-only workloads keep no top-k output: rerun it on the same scores
        import sparse_attention_amd as dsa

        got = dsa.dsa_topk(scores_t, w.index_topk, positions=None if w.positions is None else
                           w.positions.to(scores_t.device), valid_len=w.valid_len).cpu().numpy()[rows]
        check_topk_own_scores(got, ref_sc, nv[rows], w.index_topk)
        parity["topk"] = "ok"
    if step is not None:
        gpu_list = step.index_list.cpu().numpy()[rows]
        check_index_list(gpu_list, ref_list, ref_sc, nv[rows], w.index_topk, w.window)
        if not np.array_equal(np.sort(gpu_list, axis=1), np.sort(ref_list, axis=1)):
            # tied slots at the k-th score kept differently: attention parity on the step's own list
            ref_out, _ = oracle.sparse_attn(sub_aq, sub_kv, w.sink, gpu_list[:, None, :], sm_scale=w.sm_scale,
                                            dv=w.dv, nthreads=threads)
        err, rel = check_attn(step.out.float().cpu().numpy()[rows], ref_out)
        parity["index_list"] = "ok"
        parity["attention_max_abs_err"] = err
        parity["attention_max_rel_l2"] = rel
    cpu = {"value": n_slots / secs, "unit": "key-slots/s", "cores": threads, "kind": "oracle",
           "seconds": secs,
           "sample": "%d pass(es) over %d of %d sequences (%d attendable slots each pass): %s" % (
               passes, ns, w.M, n_slots // passes, "score + full-sort top-k + window union + attention"
               if step is not None else "score + full-sort top-k")}
    if step is not None:
        cpu["tokens_per_s"] = ns * passes / secs
    return cpu, parity


if __name__ == "__main__":
    main()
