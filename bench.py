#!/usr/bin/env python3
"""Throughput of blockwise exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward and one backward pass of the whole attention over one batch of
synthetic seeded input resident in HBM.  The default workload is one GPU's share of a
causal ring: B1, S8192, 16 heads of 128, bf16, 8 virtual key blocks of 1024 visited
in ring order.  Prints ONE JSON line: whole-step TFLOP/s over the algorithmic flops
(4*D per visible pair forward, 10*D backward), per-kernel HIP-event timings, the
roofline of the dominant kernel, and the oracle timed on a bounded sample on the host
cores as a CPU baseline.

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


def kernel_source_sha():
    """sha1 over the kernel sources (csrc/* and include/attn.h, sorted by name)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "ring_exact_attention_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)) + [os.path.join(root, "include", "attn.h")]
    h = hashlib.sha1()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
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


def time_segments(torch, segs, steps, warmup, stream):
    """Run warmup + timed steps of the segment list; per-segment mean ms from HIP events."""
    for _ in range(warmup):
        for _, fn in segs:
            fn()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(segs) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev = events[s]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(segs):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg_ms = {name: 0.0 for name, _ in segs}
    for ev in events:
        for i, (name, _) in enumerate(segs):
            seg_ms[name] += ev[i].elapsed_time(ev[i + 1])
    return {n: t / steps for n, t in seg_ms.items()}, wall


def copy_calibration(torch, dev, args):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    n = args.copy_bytes
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    seg_ms, _ = time_segments(torch, [("copy", lambda: b.copy_(a))], args.steps, args.warmup,
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
    seg_ms, wall = time_segments(torch, segs, args.steps, args.warmup, torch.cuda.current_stream(dev))
    slots = w.sparse_window + w.top_n * w.block_size
    gathered = B * S * slots * E * 2 * 2
    f_sparse = B * S * slots * E * 4.0
    f_select = B * 2.0 * E * w.block_size * sum(range(S // w.block_size))
    # backward per (token, slot): S and dP recomputed, dQ, dK, dV (10 E flops); it gathers
    # K, V for dq and Q, dO for dk, dv: twice the forward's gathered bytes
    f_bwd = B * S * slots * E * 10.0 if args.sparse_backward else 0.0
    ms = wall / args.steps * 1e3
    kernels = {"block_select": {"avg_us": round(seg_ms["block_select"] * 1e3, 2),
                                "fp64_gflop": round(f_select / 1e9, 3),
                                "fp64_tflops": round(f_select / (seg_ms["block_select"] * 1e-3) / 1e12, 3)},
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
        dms, _ = time_segments(torch, dsegs, args.steps, args.warmup, torch.cuda.current_stream(dev))
        step_us = (dms["decode_select"] + dms["decode_attn"]) * 1e3
        kernels["decode_step"] = {"new_tokens_per_sequence": T, "cache_rows": S,
                                  "select_us": round(dms["decode_select"] * 1e3, 2),
                                  "attn_us": round(dms["decode_attn"] * 1e3, 2), "step_us": round(step_us, 2),
                                  "tokens_per_s": round(B * T / (step_us * 1e-6), 1)}
    if args.sparse_backward:
        tb = seg_ms["attn_bwd_sparse"] * 1e-3
        kernels["attn_bwd_sparse"] = {"avg_us": round(tb * 1e6, 2), "gathered_gb": round(2 * gathered / 1e9, 3),
                                      "gathered_gbs": round(2 * gathered / tb / 1e9, 1),
                                      "tflops": round(f_bwd / tb / 1e12, 2)}
    # roofline of the dominant attention kernel (the gradient's when it is timed)
    rk = "attn_bwd_sparse" if args.sparse_backward else "attn_fwd_sparse"
    rbytes = 2 * gathered if args.sparse_backward else gathered
    ach = rbytes / (seg_ms[rk] * 1e-3) / 1e9
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
                        "traffic": measured_traffic(w.name, rk)}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = sparse_cpu_baseline(w, q, k, v, idx.cpu().numpy(), args.cpu_budget)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ring_sim_causal_s8192")
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
    q, k, v, do = workloads.generate(w, with_dout=w.backward)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dod = do.to(dev) if do is not None else None
    kw = dict(causal=w.causal, window=w.window, query_chunk=w.query_chunk, key_chunk=w.key_chunk,
              kv_block=w.kv_block)
    B, S, Hq, Hkv, D, Dv = w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dv
    sink = None
    if args.softmax == "learnable":
        sink = workloads.random_tensor((Hq,), w.seed + 100).to(dev)
    kw.update(softmax_type=args.softmax, sink=sink)
    if args.bias == "keypad":
        bias = torch.zeros((B, 1, 1, S), dtype=torch.float32, device=dev)
        bias[..., S - S // 16:] = float("-inf")
        kw.update(bias=bias)
    elif args.bias == "shared":
        kw.update(bias=workloads.random_tensor((1, 1, S, S), w.seed + 101).to(dev))
    if args.dropout > 0.0:
        # drawn on the GPU head by head (the [S, S] draws of all heads would be large)
        g = torch.Generator(device=dev).manual_seed(w.seed + 102)
        words = torch.empty((1, Hq, S, (S + 31) // 32), dtype=torch.int32, device=dev)
        for h in range(Hq):
            words[0, h] = workloads.pack_bits(torch.rand((S, S), generator=g, device=dev) < args.dropout)
        kw.update(dropout=words)
    o = torch.empty((B, S, Hq, Dv), dtype=qd.dtype, device=dev)
    m = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))
    ws = torch.empty(max(rea.bwd_workspace_bytes(qd, kd, head_dim_v=Dv, **kw), 256), dtype=torch.uint8,
                     device=dev)
    bkw = dict(kw, dsink=torch.empty((Hq,), dtype=torch.float32, device=dev)) if sink is not None else kw

    # One step, split into its kernels so each can be timed on the launch stream:
    # forward | dq (which also computes D and the LSE for the dk/dv pass) | dk,dv.
    def segments():
        yield "attn_fwd", lambda: rea.attn_fwd(qd, kd, vd, out=o, m=m, l=l, **kw)
        if w.backward:
            yield "bwd_dq", lambda: rea.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads,
                                                 skip_dkdv=True, **bkw)
            yield "bwd_dkdv", lambda: rea.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads,
                                                   skip_dq=True, reuse_stats=True, **bkw)

    segs = list(segments())
    seg_ms, wall = time_segments(torch, segs, args.steps, args.warmup, torch.cuda.current_stream(dev))

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
    # Compulsory HBM bytes per launch (bf16 tensors read or written once, fp32 stats).
    esz = 2 if w.dtype == "bf16" else 4
    qbytes, kbytes, stat = B * S * Hq * D * esz, B * S * Hkv * D * esz, B * Hq * S * 4
    obytes, vbytes = B * S * Hq * Dv * esz, B * S * Hkv * Dv * esz
    hbm = {"attn_fwd": qbytes + obytes + kbytes + vbytes + 2 * stat,
           "bwd_dq": 2 * qbytes + 2 * obytes + kbytes + vbytes + 4 * stat,
           "bwd_dkdv": qbytes + obytes + 2 * kbytes + 2 * vbytes + 2 * stat}
    kernels = {}
    for n, t in seg_ms.items():
        kernels[n] = {"avg_us": round(t * 1e3, 2), "alg_gflop": round(alg[n] / 1e9, 3),
                      "tflops": round(alg[n] / (t * 1e-3) / 1e12, 2),
                      "hbm_gbs": round(hbm[n] / (t * 1e-3) / 1e9, 1)}
    step_ms = sum(seg_ms.values())
    ms_per_step = wall / args.steps * 1e3
    total = f_fwd + f_bwd
    value = total / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = f_fwd / (seg_ms["attn_fwd"] * 1e-3) / 1e12
    bwd_ms = step_ms - seg_ms["attn_fwd"]
    bwd_tflops = f_bwd / (bwd_ms * 1e-3) / 1e12 if w.backward else None

    label = (w.name + ("" if args.softmax == "vanilla" else f"+{args.softmax}_sink")
             + ("" if args.bias == "none" else f"+{args.bias}_bias")
             + ("" if args.dropout <= 0.0 else f"+dropout{args.dropout:g}"))
    dom = max(seg_ms, key=seg_ms.get)
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(alg[dom] / (seg_ms[dom] * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(alg[dom] / (seg_ms[dom] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "avg_us": round(seg_ms[dom] * 1e3, 2), "alg_flop_per_launch": alg[dom],
            "traffic": measured_traffic(label.replace("+", "_"), dom)}
    if w.window[0] >= 0:        # sliding window: the kernels are HBM-bound
        roof.update({"bound": "hbm", "achieved": round(hbm[dom] / (seg_ms[dom] * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(hbm[dom] / (seg_ms[dom] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "alg_bytes_per_launch": hbm[dom]})

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": label,
                   "batch": B, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "head_dim_v": Dv, "causal": w.causal, "window": list(w.window),
                   "virtual_blocks": (S // w.kv_block) if w.kv_block else 1,
                   "query_chunk": w.query_chunk, "key_chunk": w.key_chunk, "parallelism": "none (1 GPU)"},
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2) if bwd_tflops else None,
        "fwd_bwd_mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_mfma_frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
