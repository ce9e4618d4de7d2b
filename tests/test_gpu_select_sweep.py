"""GPU parity of block_select over a seeded sweep of random configurations against the
fp64 oracle (bit-exact indices).

Each case draws, from its own seed, the batch, embedding (a multiple of 64 with
embed * block_size <= 32768), block size, top_n, cache length, a query range (the whole
sequence, or a few rows at an offset of the cache: decoding), and the distribution of
the inputs: Gaussian, integer-valued with repeated key blocks (exact ties), or one base
block with small offsets (near ties inside the bf16 scores' error bound).  The draws
reach both selection paths (bf16 scores with an error bound for up to 256 key blocks and
full grids; fp64 scores with candidate splits otherwise).
"""
import numpy as np
import pytest
import torch

from oracle import select

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 24


def draw(i):
    r = np.random.RandomState(7000 + i)
    bs = int(r.choice([16, 32, 64]))
    E = int(64 * r.randint(1, 1 + min(16, 32768 // bs // 64)))
    B = int(r.randint(1, 3))
    n = int(r.randint(1, 17))
    Skv = int(r.randint(bs, 4200 if bs > 16 else 2600))
    if r.rand() < 0.6:
        q_pos0, S = 0, Skv
    else:
        S = int(r.randint(1, 70))
        q_pos0 = int(r.randint(0, Skv - S + 1))
    dist = ["normal", "ties", "near"][r.randint(3)]
    return dict(B=B, E=E, bs=bs, n=n, Skv=Skv, S=S, q_pos0=q_pos0, dist=dist, seed=31 * i + 5)


def inputs(c):
    g = torch.Generator().manual_seed(c["seed"])
    B, Skv, E, bs = c["B"], c["Skv"], c["E"], c["bs"]
    if c["dist"] == "normal":
        k = torch.randn((B, Skv, E), generator=g)
        q = torch.randn((B, Skv, E), generator=g)
    elif c["dist"] == "ties":
        k = torch.randint(-2, 3, (B, Skv, E), generator=g).float()
        nb = Skv // bs
        for b in range(B):
            for blk in range(3, nb, 4):                    # block blk repeats block blk - 3
                k[b, blk * bs:(blk + 1) * bs] = k[b, (blk - 3) * bs:(blk - 2) * bs]
        q = torch.randint(-2, 3, (B, Skv, E), generator=g).float()
    else:
        base = torch.randn((bs, E), generator=g)
        nb = -(-Skv // bs)
        k = base.repeat(B, nb, 1)[:, :Skv].clone()
        for b in range(B):
            for blk in range(Skv // bs):
                k[b, blk * bs, (blk * 7 + b) % E] += ((blk * 5 + b) % 9 - 4) * 2.0 ** -7
        q = torch.randn((B, Skv, E), generator=g)
    q = q[:, c["q_pos0"]:c["q_pos0"] + c["S"]].contiguous()
    return q.to(torch.bfloat16), k.to(torch.bfloat16)


def case_id(i):
    c = draw(i)
    return f"{i}-b{c['B']}-e{c['E']}-bs{c['bs']}-n{c['n']}-kv{c['Skv']}-s{c['S']}@{c['q_pos0']}-{c['dist']}"


@pytest.mark.parametrize("i", range(N_CASES), ids=[case_id(i) for i in range(N_CASES)])
def test_select_sweep(gpu, i):
    c = draw(i)
    q, k = inputs(c)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=c["bs"], top_n=c["n"], q_pos0=c["q_pos0"])
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=c["bs"], top_n=c["n"], q_pos0=c["q_pos0"])
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
