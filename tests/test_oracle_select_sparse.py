"""Pins of the block-selection and gathered-attention oracles.

block_select: brute force with a full sort on tiny inputs (pure Python), engineered
exact ties on integer inputs, closed forms for the first blocks, exact means.
sparse_attention: K = 0 closed form (uniform weights over all slots, which pins the
zero padding, the duplicates and the -1 clamp together), constant V, and equality
with attention over an explicitly materialised candidate list built with torch ops.
sparse_attention_backward: torch autograd through that materialised list (its gather
scatters the gradients back to the sequence rows), central finite differences on a tiny
case, and the K = 0 closed forms (dq = 0; dv of a row = the sum of dO / L over the slots
that read it).
"""
import math

import numpy as np
import pytest
import torch

from oracle import select, sparse


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def brute_select(q, k, bs, n):
    B, S, E = q.shape
    out = np.full((B, S, n), -1, dtype=np.int32)
    for b in range(B):
        nb = S // bs
        means = [[sum(float(k[b, c * bs + r, e]) for r in range(bs)) / bs for e in range(E)]
                 for c in range(nb)]
        for t in range(S):
            i = t // bs
            cands = []
            for c in range(min(i, nb)):
                s = sum(float(q[b, t, e]) * means[c][e] for e in range(E))
                cands.append((-s, c))
            cands.sort()
            chosen = sorted(c for _, c in cands[:n])
            out[b, t, n - len(chosen):] = chosen
    return out


@pytest.mark.parametrize("S,bs,n,E", [(64, 8, 3, 16), (96, 8, 3, 8), (130, 16, 2, 4)])
def test_select_brute_force(S, bs, n, E):
    q, k = rnd((2, S, E), S), rnd((2, S, E), S + 1)
    np.testing.assert_array_equal(select.block_select(q, k, block_size=bs, top_n=n),
                                  brute_select(q.numpy(), k.numpy(), bs, n))


def test_select_ties_go_to_lower_index():
    bs, n, E, S = 4, 1, 4, 32
    g = torch.Generator().manual_seed(3)
    k = torch.randint(-3, 4, (1, S, E), generator=g).double()
    k[0, 12:16] = k[0, 4:8]               # block 3 duplicates block 1
    mean1 = k[0, 4:8].mean(0)
    q = (mean1 * 100).expand(1, S, E).clone()   # block 1 and 3 score highest, exactly tied
    assert float((q[0, 0] * mean1).sum()) > 0
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    for t in range(16, S):                # blocks 1 and 3 both available
        assert sel[0, t, 0] == 1, (t, sel[0, t])
    np.testing.assert_array_equal(sel, brute_select(q.numpy(), k.numpy(), bs, n))


def test_select_closed_forms_for_first_blocks():
    bs, n, E, S = 8, 4, 8, 96
    q, k = rnd((1, S, E), 5), rnd((1, S, E), 6)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    assert np.all(sel[0, :bs] == -1)                     # block 0: nothing inserted yet
    for i in range(1, n + 1):                            # fewer candidates than top_n
        for t in range(i * bs, (i + 1) * bs):
            np.testing.assert_array_equal(sel[0, t], [-1] * (n - i) + list(range(i)))
    d = np.diff(sel, axis=-1)                            # ascending; -1 padding first
    assert np.all((d > 0) | ((sel[..., :-1] == -1) & (sel[..., 1:] == -1)))


def test_block_means_exact_for_bf16_inputs():
    k = rnd((1, 64, 16), 7).to(torch.bfloat16)
    means = select.block_means(k, 32)
    kk = k.double().numpy()
    for c in range(2):
        for e in range(16):
            exact = math.fsum(kk[0, c * 32 + r, e] for r in range(32)) / 32
            assert means[0, c, e] == exact


def test_select_reports_score_gap():
    q, k = rnd((1, 128, 8), 8), rnd((1, 128, 8), 9)
    _, gap = select.block_select(q, k, block_size=8, top_n=3, return_gap=True)
    assert gap > 0


def closed_form_zero_keys(v, t, W, bs, n):
    """K = 0 => every logit is 0 and every block score ties, so token t (block i)
    selects blocks 0..min(n,i)-1 and n - min(n,i) copies of the clamped -1 block
    (bs rows of token 0); weights are uniform over W + n*bs slots."""
    i = t // bs
    keep = min(n, i)
    total = v[max(0, t - W + 1):t + 1].sum(0)
    if keep:
        total = total + v[:keep * bs].sum(0)
    total = total + (n - keep) * bs * v[0]
    return total / (W + n * bs)


def test_sparse_zero_keys_closed_form():
    B, S, E, bs, n, W = 1, 96, 8, 8, 3, 8
    q, v = rnd((B, S, E), 10), rnd((B, S, E), 11)
    k = torch.zeros((B, S, E), dtype=torch.float64)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, m, l = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    vv = v.numpy()[0]
    for t in range(S):
        np.testing.assert_allclose(o[0, t], closed_form_zero_keys(vv, t, W, bs, n), atol=1e-14, rtol=0)
    assert np.all(m == 0) and np.all(l == W + n * bs)


def test_sparse_constant_values():
    B, S, E, bs, n, W = 1, 64, 8, 8, 2, 8
    q, k = rnd((B, S, E), 12), rnd((B, S, E), 13)
    c = rnd((E,), 14)
    v = c.expand(B, S, E).clone()
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, _, _ = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    np.testing.assert_allclose(o[0, W - 1:], np.broadcast_to(c.numpy(), (S - W + 1, E)), atol=1e-13, rtol=0)


def materialised_route(q, k, v, sel, W, bs):
    return materialised_route_t(q, k, v, sel, W, bs).detach().numpy()


def materialised_route_t(q, k, v, sel, W, bs):
    """Candidate list built with tensor ops, as the page's function does: zero-padded
    windows via unfold, selected rows via index arithmetic with negatives clamped to 0,
    concatenation, einsum, softmax."""
    B, S, E = q.shape
    pad = torch.zeros((B, W - 1, E), dtype=q.dtype)
    kw = torch.cat([pad, k], 1).unfold(1, W, 1).permute(0, 1, 3, 2)    # [B, S, W, E]
    vw = torch.cat([pad, v], 1).unfold(1, W, 1).permute(0, 1, 3, 2)
    sel_t = torch.from_numpy(sel).long()                               # [B, S, n]
    items = (sel_t[..., None] * bs + torch.arange(bs)).reshape(B, S, -1)
    items = torch.where(items < 0, torch.zeros_like(items), items)
    ks = torch.stack([k[b][items[b]] for b in range(B)])
    vs = torch.stack([v[b][items[b]] for b in range(B)])
    K = torch.cat([kw, ks], 2)
    V = torch.cat([vw, vs], 2)
    s = torch.einsum("bqd,bqwd->bqw", q, K) / math.sqrt(E)
    p = torch.softmax(s, -1)
    return torch.einsum("bqw,bqwd->bqd", p, V)


def test_sparse_equals_materialised_candidate_list():
    B, S, E, bs, n, W = 2, 80, 16, 8, 3, 8
    q, k, v = rnd((B, S, E), 15), rnd((B, S, E), 16), rnd((B, S, E), 17)
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    o, _, _ = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    np.testing.assert_allclose(o, materialised_route(q, k, v, sel, W, bs), atol=1e-13, rtol=0)
    toks = [0, 5, 40, 79]
    o_s, _, _ = sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs, tokens=toks)
    np.testing.assert_array_equal(o_s[:, toks], o[:, toks])


def test_sparse_block_past_the_end_is_rejected():
    """The page's gather reads item indices inside the sequence only (its selection never
    returns a block past the last one): the oracle raises on such an index, forward and
    backward, and on a partial last block; the last full block is accepted."""
    B, S, E, bs, W = 1, 68, 8, 8, 4                # 8 full blocks and 4 rows of a ninth
    q, k, v = rnd((B, S, E), 18), rnd((B, S, E), 19), rnd((B, S, E), 20)
    nblk = S // bs
    sel = np.full((B, S, 3), -1, dtype=np.int64)
    sel[0, :, 1] = 2
    sel[0, :, 2] = nblk - 1                        # the last full block: defined
    sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
    for bad in (nblk, nblk + 5):                   # partial block, past the end
        sel[0, 10, 2] = bad
        with pytest.raises(ValueError, match="past the end"):
            sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)
        with pytest.raises(ValueError, match="past the end"):
            sparse.sparse_attention_backward(q, k, v, sel, q, window=W, block_size=bs)


@pytest.mark.parametrize("W,n", [(8, 3), (5, 2)])
def test_sparse_backward_matches_autograd_of_materialised_list(W, n):
    B, S, E, bs = 2, 72, 16, 8
    q, k, v, do = rnd((B, S, E), 21), rnd((B, S, E), 22), rnd((B, S, E), 23), rnd((B, S, E), 24)
    sel = select.block_select(q, k, block_size=bs, top_n=n)     # has -1 entries early on
    assert (sel < 0).any()
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    materialised_route_t(qt, kt, vt, sel, W, bs).backward(do)
    dq, dk, dv = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12, rtol=0)


def test_sparse_backward_finite_differences():
    B, S, E, bs, n, W = 1, 24, 4, 4, 2, 3
    q, k, v, do = (rnd((B, S, E), s).numpy() for s in (25, 26, 27, 28))
    sel = select.block_select(q, k, block_size=bs, top_n=n)
    grads = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    h = 1e-6
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + h
            lp = float((sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)[0] * do).sum())
            x[i] = old - h
            lm = float((sparse.sparse_attention(q, k, v, sel, window=W, block_size=bs)[0] * do).sum())
            x[i] = old
            num[i] = (lp - lm) / (2 * h)
        assert np.abs(num - g).max() < 1e-6 * max(1.0, np.abs(g).max())


def test_sparse_backward_zero_keys_closed_form():
    """K = 0: every logit is 0, so P = 1/L on each of the L = W + n*bs slots.  Then
    dq = scale sum_j dS_j K_j = 0, and a row p collects dv_p = sum over the slots that read
    it of dO_t / L (window slots of tokens p..p+W-1, selected slots, and for row 0 every
    slot of a -1 block)."""
    B, S, E, bs, n, W = 1, 48, 8, 8, 2, 4
    q, v, do = rnd((B, S, E), 29), rnd((B, S, E), 30), rnd((B, S, E), 31)
    k = torch.zeros((B, S, E), dtype=torch.float64)
    sel = np.full((B, S, n), -1, dtype=np.int64)
    for t in range(S):
        i = t // bs
        chosen = list(range(max(0, i - n), i))
        sel[0, t, n - len(chosen):] = chosen
    dq, dk, dv = sparse.sparse_attention_backward(q, k, v, sel, do, window=W, block_size=bs)
    L = W + n * bs
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    ref = np.zeros((S, E))
    dO = do.numpy()[0]
    for t in range(S):
        for p in range(t - W + 1, t + 1):
            if p >= 0:
                ref[p] += dO[t] / L
        for c in sel[0, t]:
            for r in range(bs):
                ref[0 if c < 0 else c * bs + r] += dO[t] / L
    np.testing.assert_allclose(dv[0], ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("T,S", [(1, 200), (3, 200), (37, 200), (1, 192), (5, 97)])
def test_decode_equals_full_sequence(T, S):
    """Decoding the last T tokens against the whole cache (q_pos0 = S - T) gives the same
    selections and outputs as the full-sequence call on those rows."""
    B, E, bs, n, W = 2, 16, 8, 3, 6
    q, k, v = rnd((B, S, E), 30 + T), rnd((B, S, E), 31 + T), rnd((B, S, E), 32 + T)
    sel_full = select.block_select(q, k, block_size=bs, top_n=n)
    sel_dec = select.block_select(q[:, S - T:], k, block_size=bs, top_n=n, q_pos0=S - T)
    np.testing.assert_array_equal(sel_dec, sel_full[:, S - T:])
    o_full, m_full, l_full = sparse.sparse_attention(q, k, v, sel_full, window=W, block_size=bs)
    o_dec, m_dec, l_dec = sparse.sparse_attention(q[:, S - T:], k, v, sel_dec, window=W, block_size=bs,
                                                  q_pos0=S - T)
    np.testing.assert_allclose(o_dec, o_full[:, S - T:], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l_dec, l_full[:, S - T:], rtol=1e-13, atol=0)


def test_decode_in_the_middle_of_the_cache_brute_force():
    """Query rows at positions 45..60 of a cache of 96 (not the end): brute-force selection
    over the full blocks before each token's block."""
    B, S, E, bs, n = 1, 96, 8, 8, 3
    q, k = rnd((B, 16, E), 40), rnd((B, S, E), 41)
    q_full = torch.zeros((B, S, E), dtype=torch.float64)
    q_full[:, 45:61] = q
    ref = brute_select(q_full.numpy(), k.numpy(), bs, n)[:, 45:61]
    np.testing.assert_array_equal(select.block_select(q, k, block_size=bs, top_n=n, q_pos0=45), ref)
