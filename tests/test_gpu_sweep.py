"""GPU parity over a seeded sweep of random dense configurations against the fp64 oracle.

Each case draws, from its own seed, a head-dim pair (32/32, 64/64, 128/128 or the MLA
pair 128/64), a GQA group, ragged lengths with Sq != Skv, a mask (causal, left window,
two-sided window, right window only, none), query / key position offsets, virtual ring
blocks whose length divides Skv (often not a multiple of 32), and optionally an additive
bias of a broadcast shape and a packed dropout array, then checks the forward outputs,
the statistics and the three gradients element by element.  The draws cover both
workgroup shapes of the forward and dq kernels and their tile boundaries.  The backward
takes the output's low part (o_lo), so that its row dot products D come from the fp32
output as in "bpt.py"; the rounded o alone carries its bf16 rounding into dq and dk,
which in one of these draws (a GQA group of 8 under a causal window of 99 keys) ends up
2% past the bf16 bound on one element of dk.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dense
from parity import check_close, check_stats

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 64
DIMS = [(32, 32), (64, 64), (128, 128), (128, 64)]


def draw(i):
    r = np.random.RandomState(9000 + i)
    D, Dv = DIMS[r.randint(len(DIMS))]
    B = int(r.randint(1, 3))
    Hkv = int(r.randint(1, 3))
    G = int(r.choice([1, 2, 4, 8, 16]))
    Hq = min(G * Hkv, 16)
    Hq -= Hq % Hkv
    if r.rand() < 0.5:                             # ring blocks of kb keys
        kb = int(r.randint(17, 201))
        Skv = kb * int(r.randint(1, 4))
    else:
        kb, Skv = 0, int(r.randint(40, 421))
    Sq = Skv if r.rand() < 0.4 else int(r.randint(20, 421))
    causal = bool(r.rand() < 0.5)
    kind = r.randint(4)
    L = int(r.randint(0, 700))
    R = int(r.randint(0, 80))
    if causal:
        window = (L, 0) if kind < 2 else (-1, -1)
    else:
        window = [(L, R), (L, -1), (-1, R), (-1, -1)][kind]
    q_pos0 = int(r.choice([0, max(Skv - Sq, 0), r.randint(0, 300)]))
    kv_pos0 = 0 if r.rand() < 0.7 else int(r.randint(0, 100))
    bias = [None, "bhij", "b11j", "1hi1"][r.randint(4)]
    pdrop = 0.0 if r.rand() < 0.6 else float(r.uniform(0.05, 0.3))
    dshape = "bhij" if r.rand() < 0.5 else "b1ij"
    return dict(D=D, Dv=Dv, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, kb=kb, causal=causal,
                window=window, q_pos0=q_pos0, kv_pos0=kv_pos0, bias=bias, pdrop=pdrop,
                dshape=dshape, seed=100 * i + 7)


def case_id(i):
    c = draw(i)
    return (f"{i}-d{c['D']}v{c['Dv']}-b{c['B']}-h{c['Hq']}x{c['Hkv']}-s{c['Sq']}x{c['Skv']}"
            f"-kb{c['kb']}-{'causal' if c['causal'] else 'full'}{c['window']}"
            f"-pos{c['q_pos0']},{c['kv_pos0']}-bias{c['bias']}-p{c['pdrop']:.2f}")


@pytest.mark.parametrize("i", range(N_CASES), ids=[case_id(i) for i in range(N_CASES)])
def test_random_config(gpu, i):
    c = draw(i)
    B, Sq, Skv, Hq, Hkv, D, Dv, s = c["B"], c["Sq"], c["Skv"], c["Hq"], c["Hkv"], c["D"], c["Dv"], c["seed"]
    t = torch.bfloat16
    q = workloads.random_tensor((B, Sq, Hq, D), s, dtype=t)
    k = workloads.random_tensor((B, Skv, Hkv, D), s + 1, dtype=t)
    v = workloads.random_tensor((B, Skv, Hkv, Dv), s + 2, dtype=t)
    do = workloads.random_tensor((B, Sq, Hq, Dv), s + 3, dtype=t)
    dims = {"b": B, "h": Hq, "i": Sq, "j": Skv, "1": 1}
    # Biases of unit scale, also for per-key offsets shared by every row ("b11j"), which
    # give a few keys most of the attention of hundreds of (row, head) pairs.  With D
    # from the fp32 output (o_lo) and P and dS as bf16 pairs in dV and dK, an fp64 model
    # of the roundings left (the result's) stays within 0.7 of 2e-2 + 2^-8 |ref| for such
    # a bias on every one of these draws.
    bias = None
    if c["bias"] is not None:
        bias = workloads.random_tensor(tuple(dims[ch] for ch in c["bias"]), s + 4)
    drop = None
    if c["pdrop"] > 0.0:
        g = torch.Generator().manual_seed(s + 5)
        drop = torch.rand(tuple(dims[ch] for ch in c["dshape"]), generator=g) < c["pdrop"]
    mask = dict(causal=c["causal"], window=c["window"], q_pos0=c["q_pos0"], kv_pos0=c["kv_pos0"])
    gk = dict(mask, kv_block=c["kb"], bias=None if bias is None else bias.to(DEV),
              dropout=None if drop is None else workloads.pack_bits(drop).to(DEV))
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o_lo = torch.empty((B, Sq, Hq, Dv), dtype=t, device=DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, o_lo=o_lo, **gk)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, o_lo=o_lo, **gk)
    torch.cuda.synchronize()
    ok = dict(mask, bias=bias, dropout=None if drop is None else drop.numpy())
    o_r, m_r, l_r = dense.forward(q, k, v, **ok)
    check_close("o", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, **ok)
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")
