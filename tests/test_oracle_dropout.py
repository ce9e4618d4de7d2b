"""Pins of the oracle's dropout ("bpt.py": a Bernoulli array over (batch, heads, q_len,
kv_len) times the dtype's most negative value joins the chunk bias, so a dropped pair
leaves the softmax and the rest are not rescaled).  The array is an input (True =
dropped), broadcastable like the bias.

* an independent library routine: torch fp64 scaled_dot_product_attention with a
  boolean attn_mask = visible and not dropped, for full and broadcast dropout shapes and
  GQA, forward and autograd gradients;
* closed forms: dropping every pair but the diagonal of a causal mask gives O = V (each
  row sees its own key only, l = 1); an all-False array changes nothing; a row whose
  pairs are all dropped gets o = 0, m = -inf, l = 0 (the reading of rows without a key).
"""
import math

import numpy as np
import pytest
import torch

from oracle import dense


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def drop_mask(shape, p, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(shape, generator=g, dtype=torch.float64) < p).numpy()


def loop_mask(S, causal, wl, wr):
    M = np.zeros((S, S), dtype=bool)
    for i in range(S):
        for j in range(S):
            M[i, j] = (not causal or j <= i) and (wr < 0 or j <= i + wr) and (wl < 0 or j >= i - wl)
    return M


def sdpa_masked(q, k, v, allowed, scale):
    """torch fp64 SDPA over the pairs allowed [B|1, H|1, S, S]; rows with no allowed pair -> 0."""
    G = q.shape[2] // k.shape[2]
    Q, K, V = (x.permute(0, 2, 1, 3) for x in (q, k, v))
    K, V = K.repeat_interleave(G, 1), V.repeat_interleave(G, 1)
    allowed = torch.from_numpy(np.broadcast_to(allowed, (Q.shape[0], Q.shape[1]) + allowed.shape[-2:]).copy())
    has = allowed.any(dim=-1, keepdim=True)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=allowed | ~has, scale=scale)
    out = torch.where(has, out, torch.zeros((), dtype=out.dtype))
    return out.permute(0, 2, 1, 3)


SHAPES = [(2, 4, 19, 19), (1, 4, 19, 19), (2, 1, 19, 19), (1, 1, 1, 19)]


@pytest.mark.parametrize("dshape", SHAPES)
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (4, 2))])
def test_dropout_matches_torch_sdpa_and_autograd(dshape, causal, window):
    B, S, Hq, Hkv, D = 2, 19, 4, 2, 8
    q, k, v, do = rnd((B, S, Hq, D), 1), rnd((B, S, Hkv, D), 2), rnd((B, S, Hkv, D), 3), rnd((B, S, Hq, D), 4)
    drop = drop_mask(dshape, 0.3, 5)
    allowed = loop_mask(S, causal, *window)[None, None] & ~drop
    scale = 1 / math.sqrt(D)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = sdpa_masked(qt, kt, vt, allowed, scale)
    out.backward(do)
    o, m, l = dense.forward(q, k, v, causal=causal, window=window, dropout=drop)
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12, rtol=0)
    dq, dk, dv = dense.backward(q, k, v, do, causal=causal, window=window, dropout=drop)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11, rtol=0)


def test_dropping_all_but_the_diagonal_returns_v():
    B, S, H, D = 1, 12, 2, 4
    q, k, v = rnd((B, S, H, D), 6), rnd((B, S, H, D), 7), rnd((B, S, H, D), 8)
    drop = ~np.eye(S, dtype=bool)[None, None]
    o, m, l = dense.forward(q, k, v, causal=True, dropout=drop)
    np.testing.assert_allclose(o, v.numpy(), atol=1e-14, rtol=0)
    np.testing.assert_allclose(l, np.ones((B, H, S)), atol=1e-14, rtol=0)


def test_no_drops_and_fully_dropped_rows():
    B, S, H, D = 2, 16, 2, 8
    q, k, v = rnd((B, S, H, D), 9), rnd((B, S, H, D), 10), rnd((B, S, H, D), 11)
    o0, m0, l0 = dense.forward(q, k, v, causal=True)
    o, m, l = dense.forward(q, k, v, causal=True, dropout=np.zeros((1, 1, S, S), dtype=bool))
    np.testing.assert_array_equal(o, o0)
    drop = np.zeros((B, H, S, S), dtype=bool)
    drop[1, 0, 7, :] = True                                 # row 7 of (b 1, head 0) loses every key
    o, m, l = dense.forward(q, k, v, causal=True, dropout=drop)
    assert np.all(o[1, 7, 0] == 0.0) and m[1, 0, 7] == -np.inf and l[1, 0, 7] == 0.0
    np.testing.assert_array_equal(np.delete(o[1], 7, axis=0), np.delete(o0[1], 7, axis=0))
