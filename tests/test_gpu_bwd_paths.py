"""GPU parity of the backward call sequences the library offers an owner of part of the
ring ("bpt.py", _ring_attention_bwd: dq stays with the query block, dk / dv travel with
the key block), and that bench.py times:

* dq alone (ATTN_BWD_SKIP_DKDV: D and the log-sum-exp computed with dq and left in the
  workspace), then dk / dv alone from those statistics (ATTN_BWD_SKIP_DQ |
  ATTN_BWD_REUSE_STATS) -- bench.py's sequence, on the full ring workload and on small
  shapes that take every kernel shape (8-wave and 4-wave dq, dk / dv with the group's
  heads split over several workgroups, the MLA head dims, a window);
* dk / dv alone without earlier statistics (ATTN_BWD_SKIP_DQ), which runs the separate
  D / log-sum-exp pass.

Each sequence must give bitwise the gradients of the single call, and match the oracle.
Every call takes the output's low part (o_lo) as bench.py's training step does.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import dense
from parity import check_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rnd(shape, seed):
    return workloads.random_tensor(shape, seed, dtype=torch.bfloat16)


def split_and_single(gpu, qd, kd, vd, o, dod, m, l, **kw):
    """(single-call grads, bench-sequence grads, skip-dq-only dk / dv)."""
    ws = torch.empty(max(gpu.bwd_workspace_bytes(qd, kd, head_dim_v=vd.shape[3], **kw), 256),
                     dtype=torch.uint8, device=DEV)
    single = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    grads = (torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")),
             torch.full_like(vd, float("nan")))
    gpu.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads, skip_dkdv=True, **kw)
    gpu.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws, out=grads, skip_dq=True, reuse_stats=True, **kw)
    ws2 = torch.full_like(ws, 255)                       # NaN bytes: nothing may be read from it
    kv_only = (torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")),
               torch.full_like(vd, float("nan")))
    gpu.attn_bwd(qd, kd, vd, o, dod, m, l, workspace=ws2, out=kv_only, skip_dq=True, **kw)
    torch.cuda.synchronize()
    return single, grads, kv_only


CASES = [
    # id, B, S, Hq, Hkv, D, Dv, causal, window, kv_block
    ("g1_ring_causal_4wave_dq", 1, 1024, 2, 2, 128, 128, True, (-1, -1), 256),
    ("g8_causal_8wave_dq_split_dkdv", 1, 640, 16, 2, 128, 128, True, (-1, -1), 0),
    ("g4_causal_split_dkdv_ragged", 2, 333, 8, 2, 128, 128, True, (-1, -1), 0),
    ("mla_128_64_gqa4_ring", 1, 512, 8, 2, 128, 64, True, (-1, -1), 128),
    ("swa100_gqa4_4wave", 1, 700, 8, 2, 128, 128, True, (100, 0), 0),
    ("d64_full_window", 1, 300, 4, 4, 64, 64, False, (40, 9), 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bench_sequence_small(gpu, case):
    name, B, S, Hq, Hkv, D, Dv, causal, window, kvb = case
    seed = zlib.crc32(name.encode()) % 10000
    q, k, v, do = rnd((B, S, Hq, D), seed), rnd((B, S, Hkv, D), seed + 1), rnd((B, S, Hkv, Dv), seed + 2), \
        rnd((B, S, Hq, Dv), seed + 3)
    kw = dict(causal=causal, window=window, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o_lo = torch.empty_like(dod)
    o, m, l = gpu.attn_fwd(qd, kd, vd, o_lo=o_lo, **kw)
    single, seq, kv_only = split_and_single(gpu, qd, kd, vd, o, dod, m, l, o_lo=o_lo, **kw)
    for nm, a, b in zip(("dq", "dk", "dv"), single, seq):
        assert torch.equal(a, b), f"{nm}: the split sequence differs from the single call"
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, causal=causal, window=window)
    check_close("dq (sequence)", seq[0], dq_r, "bf16")
    check_close("dk (sequence)", seq[1], dk_r, "bf16")
    check_close("dv (sequence)", seq[2], dv_r, "bf16")
    # dk / dv with the separate D / LSE pass
    assert torch.isnan(kv_only[0].float()).all(), "dq must be left untouched by ATTN_BWD_SKIP_DQ"
    check_close("dk (skip dq)", kv_only[1], dk_r, "bf16")
    check_close("dv (skip dq)", kv_only[2], dv_r, "bf16")


def test_bench_sequence_ring_full_size(gpu):
    """The ring workload (B1 S8192 H16 D128 causal, 8 virtual blocks of 1024) in exactly
    the calls bench.py times: bitwise equal to the single call on every head, and equal
    to the oracle on two heads, per virtual block."""
    w = workloads.WORKLOADS["ring_sim_causal_s8192"]
    q, k, v, do = workloads.generate(w)
    kw = dict(causal=w.causal, window=w.window, query_chunk=w.query_chunk, key_chunk=w.key_chunk,
              kv_block=w.kv_block)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o_lo = torch.empty_like(dod)
    o, m, l = gpu.attn_fwd(qd, kd, vd, o_lo=o_lo, **kw)
    single, seq, kv_only = split_and_single(gpu, qd, kd, vd, o, dod, m, l, o_lo=o_lo, **kw)
    for nm, a, b in zip(("dq", "dk", "dv"), single, seq):
        assert torch.equal(a, b), f"{nm}: the split sequence differs from the single call"
    bh = [5, 14]
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, heads=bh, causal=w.causal, window=w.window)
    blk = w.kv_block
    check_close("dq", seq[0][:, :, bh], dq_r[:, :, bh], "bf16", blocks=blk)
    check_close("dk", seq[1][:, :, bh], dk_r[:, :, bh], "bf16", blocks=blk)      # G = 1
    check_close("dv", seq[2][:, :, bh], dv_r[:, :, bh], "bf16", blocks=blk)
    check_close("dk (skip dq)", kv_only[1][:, :, bh], dk_r[:, :, bh], "bf16", blocks=blk)
    check_close("dv (skip dq)", kv_only[2][:, :, bh], dv_r[:, :, bh], "bf16", blocks=blk)
