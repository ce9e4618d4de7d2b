#!/usr/bin/env python3
"""Throughput of blockwise exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward and one backward pass of the whole attention over one batch of
synthetic seeded input resident in HBM.  The default workload is one GPU's share of a
causal ring: B1, S8192, 16 heads of 128, bf16, 8 virtual key blocks of 1024 visited
in ring order.  Prints ONE JSON line: whole-step TFLOP/s over the algorithmic flops
(4*D per visible pair forward, 10*D backward), per-kernel HIP-event timings (mean,
median, min), the rooflines of the dominant kernel, of the forward and of the whole
backward, and the oracle timed on a bounded sample on the host cores as a CPU baseline.
The default run also measures the other workloads under "workloads", each with its own
rooflines: GQA-16 + sliding window (fwd + bwd, HBM-bound; the 256 MiB MALL is flushed by
writing 512 MiB before every step, outside the timed events), the long-context causal
forward, and the block-sparse selection + gathered attention (MALL flushed too). The HBM
rooflines also give their fraction of the bandwidth a plain 1 GiB device copy reaches on
the same box ("reachable_copy_gbs", "frac_measured_peak"), beside the published peak.

Only one GPU is used: a run asking for more exits with a message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd, fwd+bwd) bf16 + % of MFMA peak at 1 GPU"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
PEAK_FP64_TFLOPS = 78.6          # MI355X fp64 (MFMA), published
DEFAULT_WORKLOAD = "ring_sim_causal_s8192"


def kernel_source_sha():
    """sha1 over the kernel sources (csrc/* and include/attn.h, sorted by name), with
    their comments and blank space taken out, so that an edit of a comment does not mark
    the measured counters as stale while any change to the code does."""
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "ring_exact_attention_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)) + [os.path.join(root, "include", "attn.h")]
    # string and character literals are kept whole; // and /* */ comments are dropped
    tok = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    h = hashlib.sha1()
    for f in files:
        with open(f, encoding="utf-8") as fh:
            text = tok.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", fh.read())
        h.update(os.path.basename(f).encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` (the config's workload label, '+'
    written '_') from the rocprofv3 FETCH_SIZE and WRITE_SIZE runs summarised in
    profiles/kernels_<workload>.md (each counter scaled by
    its reading for a plain copy of known size).  None when the file has no figure for
    it or the kernel sources have changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha()
    with open(path) as f:
        for line in f:
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
                if rec.get("kernel") == kernel and rec.get("source_sha1") == sha:
                    return rec["hbm_bytes_per_launch"]
    return None


def visible_pairs(Sq, Skv, causal, window, q_pos0=0, kv_pos0=0):
    """Visible (query, key) pairs per (batch, q head) for the causal / window mask."""
    import numpy as np
    i = np.arange(Sq, dtype=np.int64) + q_pos0
    lo = np.full(Sq, kv_pos0, dtype=np.int64)
    hi = np.full(Sq, kv_pos0 + Skv - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if window[1] >= 0:
        hi = np.minimum(hi, i + window[1])
    if window[0] >= 0:
        lo = np.maximum(lo, i - window[0])
    return int(np.maximum(hi - lo + 1, 0).sum())


def cpu_baseline(w, q, k, v, do, budget_s):
    """The oracle (numpy fp64) on whole heads of the same workload until ~budget_s."""
    import numpy as np
    from oracle import dense
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    pairs = visible_pairs(w.seqlen, w.seqlen, w.causal, w.window)
    heads_done, flops, t0 = 0, 0.0, time.perf_counter()
    for h in range(w.num_q_heads):
        dense.forward(q[:1], k[:1], v[:1], causal=w.causal, window=w.window, heads=[h])
        if w.backward:
            dense.backward(q[:1], k[:1], v[:1], do[:1], causal=w.causal, window=w.window, heads=[h])
        heads_done += 1
        D, Dv = w.head_dim, w.dv
        flops += ((8.0 * D + 6.0 * Dv) if w.backward else (2.0 * D + 2.0 * Dv)) * pairs
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    what = "fwd+bwd" if w.backward else "fwd"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"oracle {what} (numpy fp64) of {heads_done} of {w.num_q_heads} q heads of batch 0 "
                      f"at full length S={w.seqlen}; TFLOP/s over the same algorithmic flops as the GPU"}


def time_segments(torch, segs, steps, warmup, stream, flush=None):
    """Run warmup + timed steps of the segment list (each step runs every segment in order).
    Returns per-segment mean ms (HIP events on the launch stream), the wall time of the timed
    steps, and per-segment lists of per-step ms.  ``flush`` (the MALL flush of HBM-bound
    workloads) runs before every step, outside the events."""
    for _ in range(warmup):
        if flush is not None:
            flush()
        for _, fn in segs:
            fn()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(segs) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush()
        ev = events[s]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(segs):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: [ev[i].elapsed_time(ev[i + 1]) for ev in events] for i, (name, _) in enumerate(segs)}
    seg_ms = {n: sum(v) / len(v) for n, v in per.items()}
    return seg_ms, wall, per


def stats_us(ms_list):
    """mean / median / min of per-step times (ms) in microseconds."""
    v = sorted(ms_list)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"mean": round(sum(v) / n * 1e3, 2), "median": round(med * 1e3, 2), "min": round(v[0] * 1e3, 2)}


def mall_flusher(torch, dev, nbytes=512 << 20):
    """Writes a 512 MiB buffer: evicts the inputs of the previous step from the 256 MiB MALL
    (and the L2s) so that an HBM-bound step reads them from HBM again."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return lambda: buf.zero_()


def reachable_copy_gbs(torch, dev, nbytes=1 << 30, reps=10):
    """HBM bandwidth a plain device-to-device copy reaches on this machine (read + write bytes
    over time, median of `reps`): the practical ceiling of an HBM-bound kernel, reported
    beside the published 8 TB/s."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9


def with_measured_peak(roof, copy_gbs):
    """Adds the fraction of the reachable copy bandwidth to an HBM roofline entry."""
    if roof and roof.get("bound") == "hbm" and copy_gbs:
        roof = dict(roof)
        roof["measured_peak"] = round(copy_gbs, 1)
        roof["frac_measured_peak"] = round(roof["achieved"] / copy_gbs, 4)
    return roof


def copy_calibration(torch, dev, args):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    n = args.copy_bytes
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    seg_ms, _, _ = time_segments(torch, [("copy", lambda: b.copy_(a))], args.steps, args.warmup,
                                 torch.cuda.current_stream(dev))
    print(json.dumps({"copy_bytes": n, "avg_us": round(seg_ms["copy"] * 1e3, 2),
                      "gbs": round(2 * n / (seg_ms["copy"] * 1e-3) / 1e9, 1)}), flush=True)


def sparse_cpu_baseline(w, q, k, v, sel, budget_s):
    import numpy as np
    from oracle import select, sparse
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    E = w.head_dim
    t0 = time.perf_counter()
    select.block_select(q[:1], k[:1], block_size=w.block_size, top_n=w.top_n)
    t_sel = time.perf_counter() - t0
    sel_flops = 2.0 * E * w.block_size * sum(range(w.seqlen // w.block_size))
    slots = w.sparse_window + w.top_n * w.block_size
    toks, t1 = 0, time.perf_counter()
    step = 64
    while time.perf_counter() - t1 < budget_s and toks < w.seqlen:
        sparse.sparse_attention(q[:1], k[:1], v[:1], sel[:1], window=w.sparse_window,
                                block_size=w.block_size, tokens=range(toks, min(toks + step, w.seqlen)))
        toks = min(toks + step, w.seqlen)
    t_sp = time.perf_counter() - t1
    gathered = toks * slots * E * 2 * 2
    return {"value": round(gathered / t_sp / 1e9, 4), "unit": "GB/s gathered", "cores": int(threads),
            "host_cpus": os.cpu_count(), "kind": "oracle", "seconds": round(t_sel + t_sp, 2),
            "select_tflops": round(sel_flops / t_sel / 1e12, 6),
            "sample": f"oracle block_select of batch 0 (full S={w.seqlen}) and oracle sparse attention of "
                      f"its first {toks} tokens (numpy fp64)"}


def bench_sparse(torch, rea, workloads, w, dev, args):
    """Block selection + gathered sparse attention (one step = both), and with
    --sparse-backward its gradient too."""
    q, k, v, _ = workloads.generate(w, with_dout=False)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, S, E = w.batch, w.seqlen, w.head_dim
    idx = torch.empty((B, S, w.top_n), dtype=torch.int32, device=dev)
    o = torch.empty_like(qd)
    m = torch.empty((B, S), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    state = {}

    def fwd():
        state["o"], state["m"], state["l"] = rea.attn_fwd_sparse(qd, kd, vd, idx, window=w.sparse_window,
                                                                 block_size=w.block_size, out=o)
    segs = [("block_select", lambda: rea.block_select(qd, kd, block_size=w.block_size, top_n=w.top_n, out=idx)),
            ("attn_fwd_sparse", fwd)]
    if args.sparse_backward:
        dod = workloads.random_tensor(q.shape, w.seed + 50, dtype=torch.bfloat16).to(dev)
        grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))
        segs.append(("attn_bwd_sparse", lambda: rea.attn_bwd_sparse(
            qd, kd, vd, idx, o, dod, state["m"], state["l"], window=w.sparse_window, block_size=w.block_size,
            out=grads)))
    flush = mall_flusher(torch, dev)
    seg_ms, wall, per = time_segments(torch, segs, args.steps, args.warmup, torch.cuda.current_stream(dev),
                                      flush=flush)
    slots = w.sparse_window + w.top_n * w.block_size
    gathered = B * S * slots * E * 2 * 2
    f_sparse = B * S * slots * E * 4.0
    f_select = B * 2.0 * E * w.block_size * sum(range(S // w.block_size))
    # backward per (token, slot): S and dP recomputed, dQ, dK, dV (10 E flops); it gathers
    # K, V for dq and Q, dO for dk, dv: twice the forward's gathered bytes
    f_bwd = B * S * slots * E * 10.0 if args.sparse_backward else 0.0
    ms = wall / args.steps * 1e3
    f_sel_exec = select_exec_flops(B, S, E, w.block_size)
    kernels = {"block_select": {"avg_us": round(seg_ms["block_select"] * 1e3, 2),
                                "fp64_gflop": round(f_select / 1e9, 3),
                                "fp64_tflops": round(f_select / (seg_ms["block_select"] * 1e-3) / 1e12, 3),
                                "bf16_gflop_executed": round(f_sel_exec / 1e9, 3),
                                "bf16_tflops_executed": round(f_sel_exec / (seg_ms["block_select"] * 1e-3) / 1e12, 3)},
               "attn_fwd_sparse": {"avg_us": round(seg_ms["attn_fwd_sparse"] * 1e3, 2),
                                   "gathered_gb": round(gathered / 1e9, 3),
                                   "gathered_gbs": round(gathered / (seg_ms["attn_fwd_sparse"] * 1e-3) / 1e9, 1),
                                   "tflops": round(f_sparse / (seg_ms["attn_fwd_sparse"] * 1e-3) / 1e12, 2)}}
    if args.decode_tokens > 0:
        # decoding: T new tokens at the end of the S-row cache (selection + attention)
        T = args.decode_tokens
        qn = qd[:, S - T:].contiguous()
        idn = torch.empty((B, T, w.top_n), dtype=torch.int32, device=dev)
        on = torch.empty_like(qn)
        wsd = torch.empty(max(rea.fwd_sparse_workspace_bytes(B, T, top_n=w.top_n, window=w.sparse_window,
                                                             block_size=w.block_size, seqlen_kv=S,
                                                             q_pos0=S - T), 256), dtype=torch.uint8, device=dev)
        dsegs = [("decode_select", lambda: rea.block_select(qn, kd, block_size=w.block_size, top_n=w.top_n,
                                                            out=idn, q_pos0=S - T)),
                 ("decode_attn", lambda: rea.attn_fwd_sparse(qn, kd, vd, idn, window=w.sparse_window,
                                                             block_size=w.block_size, out=on, q_pos0=S - T,
                                                             workspace=wsd))]
        # the same selection with the cache's block means kept in the workspace from a first
        # call (the blocks before the new tokens' block; the rest are recomputed each step)
        wss = torch.empty(max(rea.select_workspace_bytes(B, T, E, block_size=w.block_size, top_n=w.top_n,
                                                         seqlen_kv=S, q_pos0=S - T), 256),
                          dtype=torch.uint8, device=dev)
        rea.block_select(qn, kd, block_size=w.block_size, top_n=w.top_n, out=idn, q_pos0=S - T, workspace=wss)
        cached = (S - T) // w.block_size
        dsegs.append(("decode_select_cached", lambda: rea.block_select(
            qn, kd, block_size=w.block_size, top_n=w.top_n, out=idn, q_pos0=S - T, workspace=wss,
            means_cached=cached)))
        dms, _, _ = time_segments(torch, dsegs, args.steps, args.warmup, torch.cuda.current_stream(dev))
        step_us = (dms["decode_select"] + dms["decode_attn"]) * 1e3
        step_c = (dms["decode_select_cached"] + dms["decode_attn"]) * 1e3
        kernels["decode_step"] = {"new_tokens_per_sequence": T, "cache_rows": S,
                                  "select_us": round(dms["decode_select"] * 1e3, 2),
                                  "attn_us": round(dms["decode_attn"] * 1e3, 2), "step_us": round(step_us, 2),
                                  "tokens_per_s": round(B * T / (step_us * 1e-6), 1),
                                  "means_cached_blocks": cached,
                                  "select_cached_us": round(dms["decode_select_cached"] * 1e3, 2),
                                  "step_cached_us": round(step_c, 2),
                                  "tokens_per_s_cached": round(B * T / (step_c * 1e-6), 1)}
    if args.sparse_backward:
        tb = seg_ms["attn_bwd_sparse"] * 1e-3
        kernels["attn_bwd_sparse"] = {"avg_us": round(tb * 1e6, 2), "gathered_gb": round(2 * gathered / 1e9, 3),
                                      "gathered_gbs": round(2 * gathered / tb / 1e9, 1),
                                      "tflops": round(f_bwd / tb / 1e12, 2)}
    for n in per:
        kernels.setdefault(n, {})["us"] = stats_us(per[n])
    # roofline of the dominant attention kernel (the gradient's when it is timed): the
    # forward on the MFMA work it executes (one 32-row step per window block and distinct
    # selected block of each 32-token group), the gradient on its compulsory HBM bytes:
    # q, k, v, o, dO read and dq, dk, dv written once (8 bf16 [B, S, E] tensors), the
    # indices and m, l read, D and the LSE written and read back (fp32 per token).  Its
    # gathered bytes (every slot's K and V rows, twice) count blocks shared within a token
    # group once per token, so they exceed what HBM can move and are reported beside it.
    rk = "attn_bwd_sparse" if args.sparse_backward else "attn_fwd_sparse"
    sp = B * S * E * 2
    rbytes = (8 * sp + B * S * (w.top_n * 4 + 8 + 16)) if args.sparse_backward else gathered
    ach = rbytes / (seg_ms[rk] * 1e-3) / 1e9
    gathered_logical = (2 * gathered if args.sparse_backward else gathered) / (seg_ms[rk] * 1e-3) / 1e9
    f_exec, nsteps = sparse_union_flops(idx.cpu().numpy(), 32, w.sparse_window, w.block_size, E)
    out = {"metric": METRIC, "value": round((f_sparse + f_select + f_bwd) / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": w.name + ("+backward" if args.sparse_backward else ""), "batch": B,
                      "seq_len": S, "embed": E, "block_size": w.block_size,
                      "top_n": w.top_n, "window": w.sparse_window, "parallelism": "none (1 GPU)"},
           "kernels": kernels,
           "roofline": {"kernel": rk, "bound": "hbm", "achieved": round(ach, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                        "avg_us": round(seg_ms[rk] * 1e3, 2), "alg_bytes_per_launch": rbytes,
                        "traffic": measured_traffic(w.name, rk), "mall_flush": True,
                        "gathered_gbs_logical": round(gathered_logical, 1)}}
    if not args.sparse_backward:
        tf = f_exec / (seg_ms[rk] * 1e-3) / 1e12
        traffic = measured_traffic(w.name, rk)
        out["roofline"] = {"kernel": rk, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                           "avg_us": round(seg_ms[rk] * 1e3, 2), "executed_flop_per_launch": f_exec,
                           "union_steps": nsteps, "traffic": traffic, "mall_flush": True,
                           "gathered_gbs_logical": round(gathered_logical, 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = sparse_cpu_baseline(w, q, k, v, idx.cpu().numpy(), args.cpu_budget)
    print(json.dumps(out), flush=True)


def dense_measure(torch, rea, workloads, w, dev, steps, warmup, softmax="vanilla", bias="none", dropout=0.0,
                  flush=None):
    """Time one dense workload: forward, then (with a backward) dq with SKIP_DKDV and dk, dv
    with SKIP_DQ | REUSE_STATS, each on the launch stream.  Returns timings (mean, median,
    min per kernel and per step), algorithmic flops and compulsory bytes per launch, and the
    rooflines of the forward, of the whole backward and of the dominant kernel."""
    q, k, v, do = workloads.generate(w, with_dout=w.backward)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dod = do.to(dev) if do is not None else None
    del q, k, v, do
    kw = dict(causal=w.causal, window=w.window, query_chunk=w.query_chunk, key_chunk=w.key_chunk,
              kv_block=w.kv_block)
    B, S, Hq, Hkv, D, Dv = w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dv
    sink = None
    if softmax == "learnable":
        sink = workloads.random_tensor((Hq,), w.seed + 100).to(dev)
    kw.update(softmax_type=softmax, sink=sink)
    if bias == "keypad":
        bt = torch.zeros((B, 1, 1, S), dtype=torch.float32, device=dev)
        bt[..., S - S // 16:] = float("-inf")
        kw.update(bias=bt)
    elif bias == "shared":
        kw.update(bias=workloads.random_tensor((1, 1, S, S), w.seed + 101).to(dev))
    if dropout > 0.0:
        # drawn on the GPU head by head (the [S, S] draws of all heads would be large)
        g = torch.Generator(device=dev).manual_seed(w.seed + 102)
        words = torch.empty((1, Hq, S, (S + 31) // 32), dtype=torch.int32, device=dev)
        for h in range(Hq):
            words[0, h] = workloads.pack_bits(torch.rand((S, S), generator=g, device=dev) < dropout)
        kw.update(dropout=words)
    if flush is None and w.window[0] >= 0:
        flush = mall_flusher(torch, dev)       # HBM-bound: every step reads its inputs from HBM
    o = torch.empty((B, S, Hq, Dv), dtype=qd.dtype, device=dev)
    m = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    # A training step keeps the output's low part for the backward's D (the fp32 output,
    # as the page's backward takes it); a forward-only workload has no use for it.
    o_lo = torch.empty_like(o) if w.backward else None
    segs = [("attn_fwd", lambda: rea.attn_fwd(qd, kd, vd, out=o, m=m, l=l, o_lo=o_lo, **kw))]
    if w.backward:
        grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))
        ws = torch.empty(max(rea.bwd_workspace_bytes(qd, kd, head_dim_v=Dv, **kw), 256), dtype=torch.uint8,
                         device=dev)
        bkw = dict(kw, o_lo=o_lo)
        if sink is not None:
            bkw["dsink"] = torch.empty((Hq,), dtype=torch.float32, device=dev)
        # dq also computes D and the LSE, which the dk/dv call takes from the workspace
        segs.append(("bwd_dq", lambda: rea.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads,
                                                    skip_dkdv=True, **bkw)))
        segs.append(("bwd_dkdv", lambda: rea.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads,
                                                      skip_dq=True, reuse_stats=True, **bkw)))
    seg_ms, wall, per = time_segments(torch, segs, steps, warmup, torch.cuda.current_stream(dev), flush=flush)

    pairs = visible_pairs(S, S, w.causal, w.window) * B * Hq
    # Per visible pair: S = Q K^T costs 2D flops and each product with V or dO 2Dv
    # (D = Dv except for the MLA head dims): forward 2D + 2Dv (= 4D); backward recompute
    # of S (2D) and dP (2Dv), dV (2Dv), dK (2D), dQ (2D) = 6D + 4Dv (= 10D).
    f_fwd = (2.0 * D + 2.0 * Dv) * pairs
    f_bwd = (6.0 * D + 4.0 * Dv) * pairs if w.backward else 0.0
    # Algorithmic flops per kernel launch: the dk/dv kernel does the recompute of S and
    # dP plus dV and dK (4D + 4Dv per pair); the dq kernel's share is dQ (2D per pair),
    # its own recompute being the cost of computing dq without atomics.
    alg = {"attn_fwd": f_fwd, "bwd_dq": 2.0 * D * pairs, "bwd_dkdv": (4.0 * D + 4.0 * Dv) * pairs}
    # Compulsory HBM bytes per launch (bf16 tensors read or written once, fp32 stats), and
    # of the whole backward (q, o, dO, k, v read, dq, dk, dv written, m, l read).
    esz = 2 if w.dtype == "bf16" else 4
    qbytes, kbytes, stat = B * S * Hq * D * esz, B * S * Hkv * D * esz, B * Hq * S * 4
    obytes, vbytes = B * S * Hq * Dv * esz, B * S * Hkv * Dv * esz
    # (o_lo, when kept, is one more o-sized write in the forward and read in the dq call.)
    lo = obytes if o_lo is not None else 0
    hbm = {"attn_fwd": qbytes + obytes + lo + kbytes + vbytes + 2 * stat,
           "bwd_dq": 2 * qbytes + 2 * obytes + lo + kbytes + vbytes + 4 * stat,
           "bwd_dkdv": qbytes + obytes + 2 * kbytes + 2 * vbytes + 2 * stat}
    hbm_bwd = 2 * qbytes + 2 * obytes + lo + 2 * kbytes + 2 * vbytes + 2 * stat
    kernels = {}
    for n, t in seg_ms.items():
        kernels[n] = {"avg_us": round(t * 1e3, 2), "us": stats_us(per[n]), "alg_gflop": round(alg[n] / 1e9, 3),
                      "tflops": round(alg[n] / (t * 1e-3) / 1e12, 2),
                      "hbm_gbs": round(hbm[n] / (t * 1e-3) / 1e9, 1)}
    step_per = [sum(per[n][i] for n in per) for i in range(steps)]
    bwd_ms = sum(seg_ms[n] for n in seg_ms if n != "attn_fwd")
    label = (w.name + ("" if softmax == "vanilla" else f"+{softmax}_sink")
             + ("" if bias == "none" else f"+{bias}_bias") + ("" if dropout <= 0.0 else f"+dropout{dropout:g}"))
    tlabel = label.replace("+", "_")
    hbm_bound = w.window[0] >= 0        # sliding window: HBM-bound

    def roofline(name, t_ms, flop, nbytes, traffic):
        r = {"kernel": name, "avg_us": round(t_ms * 1e3, 2), "traffic": traffic}
        if hbm_bound:
            ach = nbytes / (t_ms * 1e-3) / 1e9
            r.update({"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(ach / PEAK_HBM_GBS, 4), "alg_bytes_per_launch": nbytes})
        else:
            ach = flop / (t_ms * 1e-3) / 1e12
            r.update({"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(ach / PEAK_BF16_TFLOPS, 4), "alg_flop_per_launch": flop})
        return r

    dom = max(seg_ms, key=seg_ms.get)
    roof = roofline(dom, seg_ms[dom], alg[dom], hbm[dom], measured_traffic(tlabel, dom))
    roof_fwd = roofline("attn_fwd", seg_ms["attn_fwd"], f_fwd, hbm["attn_fwd"], measured_traffic(tlabel, "attn_fwd"))
    roof_bwd = None
    if w.backward:
        tq, tk = measured_traffic(tlabel, "bwd_dq"), measured_traffic(tlabel, "bwd_dkdv")
        roof_bwd = roofline("bwd_dq+bwd_dkdv", bwd_ms, f_bwd, hbm_bwd, (tq + tk) if tq and tk else None)
    return {
        "ms_per_step": wall / steps * 1e3,
        "step_us": stats_us(step_per),
        "total_flop": f_fwd + f_bwd,
        "fwd_tflops": round(f_fwd / (seg_ms["attn_fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if w.backward else None,
        "config": {"workload": label, "batch": B, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "head_dim_v": Dv, "causal": w.causal, "window": list(w.window),
                   "virtual_blocks": (S // w.kv_block) if w.kv_block else 1,
                   "query_chunk": w.query_chunk, "key_chunk": w.key_chunk, "parallelism": "none (1 GPU)"},
        "kernels": kernels,
        "roofline": roof,
        "roofline_fwd": roof_fwd,
        "roofline_bwd": roof_bwd,
        "mall_flush": flush is not None,
    }


def sparse_union_flops(sel, tokens_per_group=32, window=32, block_size=32, embed=512):
    """MFMA flops the gathered-attention kernel executes: per group of 32 consecutive
    tokens, every 32-row step (the window's blocks, then each distinct selected block,
    -1 entries counting as one) costs 32 x 32 x E x 2 for the scores and as much for P V."""
    import numpy as np
    B, S, n = sel.shape
    G = S // tokens_per_group
    g = sel[:, :G * tokens_per_group].reshape(B, G, tokens_per_group * n)
    srt = np.sort(g, axis=2)
    distinct = 1 + (np.diff(srt, axis=2) != 0).sum(axis=2)
    nwin = (window + tokens_per_group - 1 + 31) // 32
    steps = int((distinct + nwin).sum()) * ((block_size + 31) // 32)
    return steps * 32 * 32 * embed * 4.0, steps


def extra_workloads(torch, rea, workloads, dev, args):
    """The other workloads the method is measured on, each with its own roofline: GQA-16 +
    sliding window (fwd + bwd, HBM-bound, MALL flushed before every step), the long-context
    causal forward (MFMA-bound) and the block-sparse selection + gathered attention (MALL
    flushed before every step)."""
    out = {}
    copy_gbs = reachable_copy_gbs(torch, dev)
    out["reachable_copy_gbs"] = round(copy_gbs, 1)
    w3 = workloads.WORKLOADS["gqa16_swa128_s4096"]
    r3 = dense_measure(torch, rea, workloads, w3, dev, args.steps, args.warmup)     # flushes the MALL
    out[w3.name] = {"mall_flush": r3["mall_flush"], "step_us": r3["step_us"], "fwd_tflops": r3["fwd_tflops"],
                    "bwd_tflops": r3["bwd_tflops"],
                    "fwd_bwd_tflops": round(r3["total_flop"] / (r3["step_us"]["mean"] * 1e-6) / 1e12, 2),
                    "kernels": r3["kernels"], "roofline_fwd": with_measured_peak(r3["roofline_fwd"], copy_gbs),
                    "roofline_bwd": with_measured_peak(r3["roofline_bwd"], copy_gbs)}
    torch.cuda.empty_cache()
    w4 = workloads.WORKLOADS["long_causal_s131072"]
    r4 = dense_measure(torch, rea, workloads, w4, dev, max(3, args.steps // 4), max(1, args.warmup // 4))
    out[w4.name] = {"step_us": r4["step_us"], "fwd_tflops": r4["fwd_tflops"], "kernels": r4["kernels"],
                    "roofline_fwd": r4["roofline_fwd"]}
    torch.cuda.empty_cache()
    out["block_sparse_top8_s8192"] = sparse_measure(torch, rea, workloads, dev, args.steps, args.warmup,
                                                    mall_flusher(torch, dev))
    torch.cuda.empty_cache()
    return out


def sparse_measure(torch, rea, workloads, dev, steps, warmup, flush):
    """block_select + gathered sparse forward of the block-sparse workload, MALL flushed."""
    w = workloads.WORKLOADS["block_sparse_top8_s8192"]
    q, k, v, _ = workloads.generate(w, with_dout=False)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    B, S, E = w.batch, w.seqlen, w.head_dim
    idx = torch.empty((B, S, w.top_n), dtype=torch.int32, device=dev)
    o = torch.empty_like(qd)
    segs = [("block_select", lambda: rea.block_select(qd, kd, block_size=w.block_size, top_n=w.top_n, out=idx)),
            ("attn_fwd_sparse", lambda: rea.attn_fwd_sparse(qd, kd, vd, idx, window=w.sparse_window,
                                                            block_size=w.block_size, out=o))]
    seg_ms, _, per = time_segments(torch, segs, steps, warmup, torch.cuda.current_stream(dev), flush=flush)
    f_select = B * 2.0 * E * w.block_size * sum(range(S // w.block_size))
    slots = w.sparse_window + w.top_n * w.block_size
    gathered = B * S * slots * E * 2 * 2
    f_exec, nsteps = sparse_union_flops(idx.cpu().numpy(), 32, w.sparse_window, w.block_size, E)
    t_sel, t_sp = seg_ms["block_select"] * 1e-3, seg_ms["attn_fwd_sparse"] * 1e-3
    traffic = measured_traffic(w.name, "attn_fwd_sparse")
    sel_traffic = measured_traffic(w.name, "block_select")
    roof_sp = {"kernel": "attn_fwd_sparse", "bound": "mfma", "avg_us": round(t_sp * 1e6, 2),
               "achieved": round(f_exec / t_sp / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
               "frac": round(f_exec / t_sp / 1e12 / PEAK_BF16_TFLOPS, 4), "executed_flop_per_launch": f_exec,
               "union_steps": nsteps, "traffic": traffic,
               "hbm": ({"achieved": round(traffic / t_sp / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(traffic / t_sp / 1e9 / PEAK_HBM_GBS, 4)} if traffic else None),
               "gathered_gb_logical": round(gathered / 1e9, 3),
               "gathered_gbs_logical": round(gathered / t_sp / 1e9, 1)}
    # block_select scores with bf16 MFMA (two bf16 parts of each mean) and decides the top n
    # with an error bound, scoring exactly in fp64 only the candidates within it: its
    # roofline is the bf16 work it executes; the exact fp64 scores it stands for are
    # reported beside it (their rate against the fp64 peak)
    f_sel_exec = select_exec_flops(B, S, E, w.block_size)
    roof_sel = {"kernel": "block_select", "bound": "mfma", "avg_us": round(t_sel * 1e6, 2),
                "achieved": round(f_sel_exec / t_sel / 1e12, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(f_sel_exec / t_sel / 1e12 / PEAK_BF16_TFLOPS, 4),
                "executed_flop_per_launch": f_sel_exec,
                "fp64_equivalent": {"alg_flop_per_launch": f_select, "achieved": round(f_select / t_sel / 1e12, 3),
                                    "peak": PEAK_FP64_TFLOPS,
                                    "frac": round(f_select / t_sel / 1e12 / PEAK_FP64_TFLOPS, 4)},
                "traffic": sel_traffic}
    return {"mall_flush": True, "kernels": {n: {"us": stats_us(per[n])} for n in per},
            "roofline_select": roof_sel, "roofline_sparse": roof_sp}


def select_exec_flops(B, S, E, bs, nblk=None):
    """bf16 MFMA flops block_select executes on a full sequence: query block i scores its
    min(i, nblk) candidates in tiles of 32 against 32-token tiles, two bf16 parts each."""
    nblk = S // bs if nblk is None else nblk
    tok_tiles = (bs + 31) // 32
    tiles = sum((min(i, nblk) + 31) // 32 for i in range(S // bs))
    return B * tiles * tok_tiles * 2 * (2.0 * 32 * 32 * E)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--decode-tokens", type=int, default=0,
                    help="block-sparse workload: also time decoding this many new tokens per sequence "
                         "against the full cache (selection + attention)")
    ap.add_argument("--sparse-backward", action="store_true",
                    help="block-sparse workload: also time the gradient (attn_bwd with sel_idx)")
    ap.add_argument("--softmax", default="vanilla", choices=["vanilla", "off_by_one", "learnable"],
                    help="sink softmax variant of the dense workloads (learnable: seeded N(0,1) logits)")
    ap.add_argument("--bias", default="none", choices=["none", "keypad", "shared"],
                    help="additive logit bias: keypad = [B,1,1,S] with the last S/16 keys at -inf, "
                         "shared = one random [1,1,S,S] fp32 matrix")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability: a seeded Bernoulli array [1, Hq, S, S], packed, "
                         "removes the dropped pairs from the softmax")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run only: skip the other workloads (GQA-16 SWA, long context, block-sparse)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the kernels run on one GPU's share and no multi-GPU path is provided.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import ring_exact_attention_amd as rea

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    rea.lib()                                         # fail loudly if libattn.so is missing
    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.copy_bytes:
        return copy_calibration(torch, dev, args)
    if w.sparse:
        return bench_sparse(torch, rea, workloads, w, dev, args)
    res = dense_measure(torch, rea, workloads, w, dev, args.steps, args.warmup, softmax=args.softmax,
                        bias=args.bias, dropout=args.dropout)
    value = res["total_flop"] / (res["ms_per_step"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": res["config"],
        "step_us": res["step_us"],
        "fwd_tflops": res["fwd_tflops"],
        "bwd_tflops": res["bwd_tflops"],
        "fwd_bwd_mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_mfma_frac": round(res["fwd_tflops"] / PEAK_BF16_TFLOPS, 4),
        "kernels": res["kernels"],
        "roofline": res["roofline"],
        "roofline_fwd": res["roofline_fwd"],
        "roofline_bwd": res["roofline_bwd"],
    }
    default_run = (args.workload == DEFAULT_WORKLOAD and args.softmax == "vanilla" and args.bias == "none"
                   and args.dropout <= 0.0)
    if not args.no_cpu_baseline:
        q, k, v, do = workloads.generate(w, with_dout=w.backward)
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, args.cpu_budget)
        del q, k, v, do
    if default_run and not args.no_extras:
        out["workloads"] = extra_workloads(torch, rea, workloads, dev, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
