"""GPU parity of block_select (bit-exact indices), the gathered block-sparse forward
(attn_fwd with sel_idx) and its gradient (attn_bwd with sel_idx) against the fp64
oracle, on seeded inputs: small ragged shapes, engineered exact ties, hand-made
selections, the degenerate first blocks, and the full-size workload (B4 S8192, 8 heads
x 64 as a joint embedding of 512, top-8 of 32-token blocks, window 32)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import select, sparse
from parity import check_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rnd(shape, seed):
    return workloads.random_tensor(shape, seed, dtype=torch.bfloat16)


@pytest.mark.parametrize("B,S,E,bs,n", [(2, 256, 64, 16, 3), (1, 300, 512, 32, 8), (2, 200, 128, 64, 2),
                                         (1, 1000, 512, 32, 16), (3, 64, 64, 32, 1), (1, 700, 512, 64, 5),
                                         (1, 520, 1024, 16, 16), (1, 600, 1024, 32, 8)])
def test_select_small(gpu, B, S, E, bs, n):
    q, k = rnd((B, S, E), S + E), rnd((B, S, E), S + E + 1)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


def test_select_exact_ties(gpu):
    """Integer-valued inputs with duplicated key blocks: every tie must go to the lower index."""
    B, S, E, bs, n = 2, 512, 64, 32, 3
    g = torch.Generator().manual_seed(5)
    k = torch.randint(-2, 3, (B, S, E), generator=g).to(torch.bfloat16)
    for b in range(B):
        for c in range(4, S // bs, 3):
            k[b, c * bs:(c + 1) * bs] = k[b, (c - 3) * bs:(c - 2) * bs]     # block c repeats block c-3
    q = torch.randint(-2, 3, (B, S, E), generator=g).to(torch.bfloat16)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("n", [1, 2])
def test_select_scores_equal_in_fp32(gpu, n):
    """Scores that differ only below fp32 resolution (block 7 = block 3 plus 2^-30 in one
    dimension, block 9 = block 3): the first chunk's cut is taken on fp32-rounded scores,
    so all three pass it and the exact ranking must put 7 first, then 3 before 9."""
    B, S, E, bs = 1, 384, 64, 32
    g = torch.Generator().manual_seed(11)
    k = (torch.randint(-2, 3, (B, S, E), generator=g).float() * 2.0 ** -6).to(torch.bfloat16)
    base = torch.zeros(E)
    base[0] = 1.0
    base[2] = 0.5
    for c, extra in ((3, 0.0), (7, 2.0 ** -30), (9, 0.0)):
        row = base.clone()
        row[1] = extra
        k[0, c * bs:(c + 1) * bs] = row.to(torch.bfloat16)
    q = (torch.randint(-2, 3, (B, S, E), generator=g).float() * 2.0 ** -6).to(torch.bfloat16)
    q[0, :, 0] = 1.0
    q[0, :, 1] = 1.0
    q[0, :, 2] = 1.0
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    last = ref[0, -1]                                  # a token of the last query block
    assert list(last) == ([7] if n == 1 else [3, 7])


@pytest.mark.parametrize("n,bs", [(3, 32), (8, 32), (16, 32), (3, 16), (16, 16)])
def test_select_split_candidates_ties(gpu, n, bs):
    """Few query blocks against a long cache.  With 32-row blocks (256 candidates) each
    query block's scores fit one workgroup (approximate scores, exact ones near the cut);
    with 16-row blocks (512) the candidates are shared out over several workgroups (fp64
    scores, running lists) and their lists merged.  Integer-valued inputs with repeated
    key blocks put exact ties across the shares; the indices must equal the oracle's and
    the full-sequence call's."""
    B, S, E, T, pos0 = 2, 8192, 64, 100, 8000
    g = torch.Generator().manual_seed(40 + n)
    k = torch.randint(-2, 3, (B, S, E), generator=g).to(torch.bfloat16)
    for b in range(B):
        for c in range(70, S // bs, 67):
            k[b, c * bs:(c + 1) * bs] = k[b, (c - 69) * bs:(c - 68) * bs]   # block c repeats block c-69
    q = torch.randint(-2, 3, (B, S, E), generator=g).to(torch.bfloat16)
    qn = q[:, pos0:pos0 + T].contiguous()
    idx = gpu.block_select(qn.to(DEV), k.to(DEV), block_size=bs, top_n=n, q_pos0=pos0)
    idx_full = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(qn, k, block_size=bs, top_n=n, q_pos0=pos0)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_full.cpu().numpy()[:, pos0:pos0 + T])


@pytest.mark.parametrize("scale", [0.0, 2.0 ** 70])
def test_select_degenerate_scores(gpu, scale):
    """All scores zero (every candidate tied: the lowest indices win), and scores past the
    fp32 range (inputs of 2^70: the approximate scores overflow, so every candidate is
    scored exactly in fp64)."""
    B, S, E, bs, n = 2, 640, 128, 32, 5
    q, k = rnd((B, S, E), 71), rnd((B, S, E), 72)
    q = (q.float() * scale).to(torch.bfloat16)
    k = (k.float() * (scale if scale > 0 else 1.0)).to(torch.bfloat16)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    if scale == 0.0:
        assert (ref[:, -1] == np.arange(n)).all()


@pytest.mark.parametrize("n,step,E", [(1, 2.0 ** -8, 256), (4, 2.0 ** -8, 256), (8, 2.0 ** -8, 256),
                                      (4, 2.0 ** -5, 256), (8, 2.0 ** -5, 256), (8, 2.0 ** -8, 1024)])
def test_select_near_ties(gpu, n, step, E):
    """Every key block is one base block plus a small offset in one dimension of one row,
    so the block means differ by multiples of step / 32 and the scores by about 10^-4
    (step 2^-8: inside the bf16 scores' error bound, every candidate is undecided and the
    exact fp64 scores rank them all) or 10^-3 (2^-5: some candidates decided, some not)."""
    B, S, bs = 2, 2048, 32
    g = torch.Generator().manual_seed(90 + n)
    base = torch.randn((bs, E), generator=g)
    k = base.repeat(B, S // bs, 1).reshape(B, S, E).clone()
    for b in range(B):
        for c in range(S // bs):
            k[b, c * bs, (c * 7 + b) % E] += ((c * 5 + b) % 9 - 4) * step
    k = k.to(torch.bfloat16)
    q = rnd((B, S, E), 95 + n)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("bs,pos0", [(32, 69), (16, 3)])
def test_select_offset_queries_full_grid(gpu, bs, pos0):
    """Query rows starting at an unaligned position of the key sequence (a partial first
    query block) with enough query blocks for one workgroup each: the bf16-bound path
    with q_pos0 > 0."""
    B, S, E, n = 1, 8192 if bs == 32 else 4096, 256, 8
    q, k = rnd((B, S, E), 120 + bs), rnd((B, S, E), 121 + bs)
    qn = q[:, pos0:].contiguous()
    idx = gpu.block_select(qn.to(DEV), k.to(DEV), block_size=bs, top_n=n, q_pos0=pos0)
    torch.cuda.synchronize()
    ref = select.block_select(qn, k, block_size=bs, top_n=n, q_pos0=pos0)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("bs", [32, 16])
def test_select_means_cached(gpu, bs):
    """Decoding with the block means kept across calls: a first call computes the means of
    the cache; the cache then gains rows (its blocks from c0 on change) and a second call
    with means_cached = c0 on the same workspace recomputes only those.  Both equal the
    oracle on their cache, and equal a call that computes every mean on a poisoned
    workspace.  (32-row blocks of 8192 rows: 256 blocks, the bf16-bound path for the full
    cache; 16-row blocks: 512, the split fp64 path.)"""
    B, S, E, n, T = 2, 8192, 128, 8, 16
    q, k = rnd((B, S, E), 130 + bs), rnd((B, S, E), 131 + bs)
    nblk = S // bs
    ws = torch.empty(gpu.lib().block_select_workspace_bytes(ctypes.byref(_sel_params(gpu, B, T, E, bs, n, S, S - T))),
                     dtype=torch.uint8, device=DEV)
    kd = k.to(DEV)
    idx_full = gpu.block_select(q.to(DEV), kd, block_size=bs, top_n=n, workspace=ws)   # every mean
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx_full.cpu().numpy(), select.block_select(q, k, block_size=bs, top_n=n))
    c0 = nblk - 40
    k2 = k.clone()
    k2[:, c0 * bs:] = rnd((B, S - c0 * bs, E), 140 + bs)        # rows of blocks >= c0 change
    qn = q[:, S - T:].contiguous()
    idx = gpu.block_select(qn.to(DEV), k2.to(DEV), block_size=bs, top_n=n, q_pos0=S - T, workspace=ws,
                           means_cached=c0)
    ws_poison = torch.full_like(ws, 0xFF)
    idx_all = gpu.block_select(qn.to(DEV), k2.to(DEV), block_size=bs, top_n=n, q_pos0=S - T, workspace=ws_poison)
    torch.cuda.synchronize()
    ref = select.block_select(qn, k2, block_size=bs, top_n=n, q_pos0=S - T)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    np.testing.assert_array_equal(idx_all.cpu().numpy(), ref)


def _sel_params(gpu, B, S, E, bs, n, skv, pos0):
    p = gpu.SelectParams()
    p.struct_size = ctypes.sizeof(gpu.SelectParams)
    p.dtype = gpu.ATTN_BF16
    p.batch, p.seqlen, p.embed, p.block_size, p.top_n = B, S, E, bs, n
    p.seqlen_kv, p.q_pos0 = skv, pos0
    return p


def test_select_many_blocks(gpu):
    """More than 256 candidate blocks with one workgroup per query block (260 blocks of 16
    rows): the fp64 running-list path without a candidate split."""
    B, S, E, bs, n = 1, 4160, 64, 16, 8
    q, k = rnd((B, S, E), 81), rnd((B, S, E), 82)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=bs, top_n=n)
    torch.cuda.synchronize()
    ref = select.block_select(q, k, block_size=bs, top_n=n)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


def test_select_full_size(gpu):
    w = workloads.WORKLOADS["block_sparse_top8_s8192"]
    q, k, v, _ = workloads.generate(w)
    idx = gpu.block_select(q.to(DEV), k.to(DEV), block_size=w.block_size, top_n=w.top_n)
    torch.cuda.synchronize()
    ref, gap = select.block_select(q, k, block_size=w.block_size, top_n=w.top_n, return_gap=True)
    print(f"smallest gap between the 8th and 9th score: {gap:.3e}")
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("B,S,bs,n,W", [(1, 200, 32, 4, 32), (2, 160, 16, 8, 7), (1, 256, 64, 2, 64),
                                        (1, 96, 32, 8, 1)])
def test_sparse_small(gpu, B, S, bs, n, W):
    E = 512
    q, k, v = rnd((B, S, E), 7 + S), rnd((B, S, E), 8 + S), rnd((B, S, E), 9 + S)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, m, l = gpu.attn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                                  window=W, block_size=bs)
    torch.cuda.synchronize()
    o_r, m_r, l_r = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    check_close("o", o, o_r, "bf16")
    np.testing.assert_allclose(m.cpu().numpy(), m_r, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy(), l_r, rtol=1e-3, atol=0)


@pytest.mark.parametrize("B,S", [(1, 2048), (2, 4100)])
def test_sparse_tokens_per_workgroup(gpu, B, S):
    """Grids where a workgroup takes 4 (S 2048) or 16 (S 4100, ragged tail) tokens and
    their shared union of blocks, between the one-token workgroups of small inputs and
    the 32-token ones of the full workload."""
    E, bs, n, W = 512, 32, 8, 32
    q, k, v = rnd((B, S, E), 17 + S), rnd((B, S, E), 18 + S), rnd((B, S, E), 19 + S)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, m, l = gpu.attn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                                  window=W, block_size=bs)
    torch.cuda.synchronize()
    o_r, m_r, l_r = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    check_close("o", o, o_r, "bf16")
    np.testing.assert_allclose(m.cpu().numpy(), m_r, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy(), l_r, rtol=1e-3, atol=0)


def test_sparse_zero_keys_uniform_weights(gpu):
    """K = 0: all logits 0, so o is the plain mean over all slots (zero pads, duplicate
    clamped rows of token 0 and all)."""
    B, S, E, bs, n, W = 1, 160, 512, 32, 8, 32
    q, v = rnd((B, S, E), 11), rnd((B, S, E), 12)
    k = torch.zeros((B, S, E), dtype=torch.bfloat16)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, m, l = gpu.attn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                                  window=W, block_size=bs)
    torch.cuda.synchronize()
    o_r, _, _ = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    check_close("o", o, o_r, "bf16")
    assert torch.all(l == W + n * bs)


def test_sparse_full_size_sampled(gpu):
    w = workloads.WORKLOADS["block_sparse_top8_s8192"]
    q, k, v, _ = workloads.generate(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idx = gpu.block_select(qd, kd, block_size=w.block_size, top_n=w.top_n)
    o, m, l = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=w.sparse_window, block_size=w.block_size)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    g = np.random.default_rng(4)
    toks = sorted(set([0, 1, 31, 32, 255, 256, 4095, w.seqlen - 1] + list(g.integers(0, w.seqlen, 24))))
    o_r, m_r, l_r = sparse.sparse_attention(q, k, v, sel, window=w.sparse_window, block_size=w.block_size,
                                            tokens=toks)
    oo = o.view(w.batch, w.seqlen, -1)
    check_close("o", oo[:, toks], o_r[:, toks], "bf16")
    np.testing.assert_allclose(m.cpu().numpy()[:, toks], m_r[:, toks], atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy()[:, toks], l_r[:, toks], rtol=1e-3, atol=0)


def handmade_selection(B, S, bs, n, seed):
    """Selections block_select never produces, all inside the sequence: duplicates within a
    token's list, several -1 entries (token 0 for every row), random order, blocks at or
    after the token's own, shared and unshared blocks across the 32-token groups."""
    g = np.random.default_rng(seed)
    nblk = S // bs
    sel = g.integers(-1, nblk, size=(B, S, n)).astype(np.int32)
    sel[:, ::5, 1] = sel[:, ::5, 0]                 # duplicates
    sel[:, ::7, :3] = -1                            # several -1
    return sel


def test_sparse_handmade_selection(gpu):
    B, S, E, bs, n, W = 2, 224, 512, 32, 6, 20
    q, k, v = rnd((B, S, E), 41), rnd((B, S, E), 42), rnd((B, S, E), 43)
    sel = handmade_selection(B, S, bs, n, 44)
    o, m, l = gpu.attn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                                  window=W, block_size=bs)
    torch.cuda.synchronize()
    o_r, m_r, l_r = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    check_close("o", o, o_r, "bf16")
    np.testing.assert_allclose(m.cpu().numpy(), m_r, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy(), l_r, rtol=1e-3, atol=0)


def test_sparse_past_the_end_contract(gpu):
    """A selected block past the last one is outside the page's definition (its selection
    never returns one; the oracle rejects it).  The kernels' contract for it: the
    range-checked reads see zero rows, nothing faults, every output is finite, and the
    result equals the same call on a sequence extended by one block of zero rows (query
    and dO rows zero too) with those indices pointing at that block.  Kernel against
    kernel, no oracle."""
    B, S, E, bs, n, W = 2, 224, 512, 32, 6, 20
    nblk = S // bs
    q, k, v, do = rnd((B, S, E), 141), rnd((B, S, E), 142), rnd((B, S, E), 143), rnd((B, S, E), 144)
    sel = handmade_selection(B, S, bs, n, 145)
    sel[:, 3::11, 4] = nblk + 7                     # past the end
    sel[:, 5::13, 2] = nblk
    z = torch.zeros((B, bs, E), dtype=torch.bfloat16)
    q2, k2, v2, do2 = (torch.cat([x, z], 1) for x in (q, k, v, do))
    sel2 = np.concatenate([np.where(sel >= nblk, nblk, sel), np.full((B, bs, n), -1, np.int32)], 1)
    sel2 = np.ascontiguousarray(sel2.astype(np.int32))
    # forward
    idx, idx2 = torch.from_numpy(sel).to(DEV), torch.from_numpy(sel2).to(DEV)
    o, m, l = gpu.attn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), idx, window=W, block_size=bs)
    o2, m2, l2 = gpu.attn_fwd_sparse(q2.to(DEV), k2.to(DEV), v2.to(DEV), idx2, window=W, block_size=bs)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(m).all() and torch.isfinite(l).all()
    check_close("o vs zero-extended", o, o2[:, :S], "bf16")
    np.testing.assert_allclose(l.cpu().numpy(), l2[:, :S].cpu().numpy(), rtol=1e-5, atol=0)
    # backward: the extra rows have q = dO = 0, so they pass nothing to dk, dv of the rest
    dq, dk, dv = sparse_grads(gpu, q, k, v, do, sel, W)
    dq2, dk2, dv2 = sparse_grads(gpu, q2, k2, v2, do2, sel2, W)
    for nm, a_, b_ in (("dq", dq, dq2), ("dk", dk, dk2), ("dv", dv, dv2)):
        assert torch.isfinite(a_.float()).all(), nm
        check_close(f"{nm} vs zero-extended", a_, b_[:, :S], "bf16")


# ---------------------------------------------------------------- backward (sel_block 32)
def sparse_grads(gpu, q, k, v, do, sel, W, bs=32):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    idx = torch.from_numpy(np.ascontiguousarray(sel)).to(DEV) if isinstance(sel, np.ndarray) else sel
    o, m, l = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=W, block_size=bs)
    grads = gpu.attn_bwd_sparse(qd, kd, vd, idx, o, dod, m, l, window=W, block_size=bs)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("B,S,n,W", [(1, 200, 4, 32), (2, 160, 8, 7), (1, 96, 8, 1), (1, 300, 8, 64),
                                     (2, 256, 16, 32), (1, 203, 8, 32), (1, 450, 12, 16)])
def test_sparse_backward_small(gpu, B, S, n, W):
    E, bs = 512, 32
    q, k, v, do = rnd((B, S, E), 60 + S), rnd((B, S, E), 61 + S), rnd((B, S, E), 62 + S), rnd((B, S, E), 63 + S)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    dq, dk, dv = sparse_grads(gpu, q, k, v, do, sel, W)
    dq_r, dk_r, dv_r = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


@pytest.mark.parametrize("S,n", [(224, 6), (203, 8)])
def test_sparse_backward_handmade_selection(gpu, S, n):
    """Duplicates, several -1 entries (all collected by row 0), tokens listing blocks at or
    after their own; top_n 8 with a token count that is not a multiple of 4 takes the
    16-byte reads of the selection with a partial last group."""
    B, E, bs, W = 2, 512, 32, 20
    q, k, v, do = rnd((B, S, E), 45), rnd((B, S, E), 46), rnd((B, S, E), 47), rnd((B, S, E), 48)
    sel = handmade_selection(B, S, bs, n, 49)
    dq, dk, dv = sparse_grads(gpu, q, k, v, do, sel, W)
    dq_r, dk_r, dv_r = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


def test_sparse_backward_zero_keys(gpu):
    B, S, E, bs, n, W = 1, 160, 512, 32, 8, 32
    q, v, do = rnd((B, S, E), 50), rnd((B, S, E), 51), rnd((B, S, E), 52)
    k = torch.zeros((B, S, E), dtype=torch.bfloat16)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    dq, dk, dv = sparse_grads(gpu, q, k, v, do, sel, W)
    dq_r, dk_r, dv_r = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    assert float(dq.abs().max()) == 0.0                       # K = 0: dq is exactly zero
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


def test_sparse_backward_full_size_batch0(gpu):
    """The full workload (B4 S8192 E512, top-8 of 32-token blocks, window 32) on the GPU;
    batch 0 checked completely against the oracle (its dk, dv depend on batch 0 only)."""
    w = workloads.WORKLOADS["block_sparse_top8_s8192"]
    q, k, v, _ = workloads.generate(w)
    do = workloads.random_tensor(q.shape, w.seed + 50, dtype=torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idx = gpu.block_select(qd, kd, block_size=w.block_size, top_n=w.top_n)
    dq, dk, dv = sparse_grads(gpu, q, k, v, do, idx, w.sparse_window)
    dq2, dk2, dv2 = sparse_grads(gpu, q, k, v, do, idx, w.sparse_window)
    for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a_, b_)                           # bitwise reproducible
    sel = idx.cpu().numpy()
    dq_r, dk_r, dv_r = sparse.sparse_attention_backward(q[:1], k[:1], v[:1], sel[:1], do[:1],
                                                        window=w.sparse_window, block_size=w.block_size)
    check_close("dq", dq[:1], dq_r, "bf16")
    check_close("dk", dk[:1], dk_r, "bf16")
    check_close("dv", dv[:1], dv_r, "bf16")


# ---------------------------------------------------------------- decoding against a cache
@pytest.mark.parametrize("S,T,pos0", [(1000, 1, 999), (1000, 4, 996), (1000, 33, 967), (1000, 20, 500),
                                      (256, 32, 224)])
def test_decode_against_cache(gpu, S, T, pos0):
    """New tokens at positions pos0 .. pos0 + T - 1 against a key / value cache of S rows:
    selection bit-exact and output within tolerance of the oracle, and the same
    selection as the full-sequence call on those rows."""
    B, E, bs, n, W = 2, 512, 32, 8, 32
    q, k, v = rnd((B, S, E), 70 + T), rnd((B, S, E), 71 + T), rnd((B, S, E), 72 + T)
    qn = q[:, pos0:pos0 + T].contiguous()
    qd, kd, vd = qn.to(DEV), k.to(DEV), v.to(DEV)
    idx = gpu.block_select(qd, kd, block_size=bs, top_n=n, q_pos0=pos0)
    o, m, l = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=W, block_size=bs, q_pos0=pos0)
    idx_full = gpu.block_select(q.to(DEV), kd, block_size=bs, top_n=n)
    torch.cuda.synchronize()
    sel = select.block_select(qn, k, block_size=bs, top_n=n, q_pos0=pos0)
    np.testing.assert_array_equal(idx.cpu().numpy(), sel)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_full.cpu().numpy()[:, pos0:pos0 + T])
    o_r, m_r, l_r = sparse.sparse_attention(qn, k, v, sel, window=W, block_size=bs, q_pos0=pos0)
    check_close("o", o, o_r, "bf16")
    np.testing.assert_allclose(m.cpu().numpy(), m_r, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy(), l_r, rtol=1e-3, atol=0)


@pytest.mark.parametrize("B,T,pos0", [(2, 1, 999), (1, 5, 700), (3, 2, 64)])
def test_decode_split_over_steps(gpu, B, T, pos0):
    """Decoding with the workspace: each token's steps are shared out over several
    workgroups and combined; equal (within rounding) to the unsplit call and to the
    oracle."""
    S, E, bs, n, W = 1000, 512, 32, 8, 32
    q, k, v = rnd((B, S, E), 90 + T), rnd((B, S, E), 91 + T), rnd((B, S, E), 92 + T)
    qn = q[:, pos0:pos0 + T].contiguous()
    qd, kd, vd = qn.to(DEV), k.to(DEV), v.to(DEV)
    assert gpu.fwd_sparse_workspace_bytes(B, T, top_n=n, seqlen_kv=S, q_pos0=pos0) > 0
    idx = gpu.block_select(qd, kd, block_size=bs, top_n=n, q_pos0=pos0)
    o, m, l = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=W, block_size=bs, q_pos0=pos0)
    o1, m1, l1 = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=W, block_size=bs, q_pos0=pos0, workspace=False)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    o_r, m_r, l_r = sparse.sparse_attention(qn, k, v, sel, window=W, block_size=bs, q_pos0=pos0)
    check_close("o (split)", o, o_r, "bf16")
    check_close("o (unsplit)", o1, o_r, "bf16")
    np.testing.assert_allclose(m.cpu().numpy(), m_r, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l.cpu().numpy(), l_r, rtol=1e-3, atol=0)
    np.testing.assert_allclose(m.cpu().numpy(), m1.cpu().numpy(), atol=1e-5, rtol=0)


def test_decode_full_size_cache(gpu):
    """One new token per sequence at the end of the full workload's 8192-row cache."""
    w = workloads.WORKLOADS["block_sparse_top8_s8192"]
    q, k, v, _ = workloads.generate(w)
    S = w.seqlen
    qn = q[:, S - 1:].contiguous()
    qd, kd, vd = qn.to(DEV), k.to(DEV), v.to(DEV)
    idx = gpu.block_select(qd, kd, block_size=w.block_size, top_n=w.top_n, q_pos0=S - 1)
    o, m, l = gpu.attn_fwd_sparse(qd, kd, vd, idx, window=w.sparse_window, block_size=w.block_size, q_pos0=S - 1)
    torch.cuda.synchronize()
    sel = select.block_select(qn, k, block_size=w.block_size, top_n=w.top_n, q_pos0=S - 1)
    np.testing.assert_array_equal(idx.cpu().numpy(), sel)
    o_r, _, _ = sparse.sparse_attention(qn, k, v, sel, window=w.sparse_window, block_size=w.block_size,
                                        q_pos0=S - 1)
    check_close("o", o, o_r, "bf16")
