"""Pins of the oracle's additive logit bias ("bpt.py": ring_attention / blockwise_attn take a
bias broadcastable to (batch, heads, q_len, kv_len), added to the scaled logits).

* an independent library routine: torch fp64 scaled_dot_product_attention with a float
  attn_mask equal to the bias on visible pairs and -inf elsewhere, for full and broadcast
  bias shapes (a key-padding bias [B, 1, 1, Skv] among them);
* torch autograd through the same routine (the bias gets no gradient on the page);
* closed forms: a bias constant along each row changes nothing; -inf on a pair is the same
  as masking it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dense


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def loop_mask(S, causal, wl, wr):
    M = np.zeros((S, S), dtype=bool)
    for i in range(S):
        for j in range(S):
            M[i, j] = (not causal or j <= i) and (wr < 0 or j <= i + wr) and (wl < 0 or j >= i - wl)
    return M


def sdpa_biased(q, k, v, bias, mask, scale):
    G = q.shape[2] // k.shape[2]
    Q, K, V = (x.permute(0, 2, 1, 3) for x in (q, k, v))
    K, V = K.repeat_interleave(G, 1), V.repeat_interleave(G, 1)
    m = torch.where(torch.from_numpy(mask), torch.zeros((), dtype=q.dtype), torch.full((), float("-inf"), dtype=q.dtype))
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=m + bias, scale=scale)
    return out.permute(0, 2, 1, 3)


SHAPES = [(2, 4, 19, 19), (1, 4, 19, 19), (2, 1, 1, 19), (1, 1, 19, 1), (2, 4, 1, 19)]


@pytest.mark.parametrize("bshape", SHAPES)
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (4, 2))])
def test_bias_matches_torch_sdpa_and_autograd(bshape, causal, window):
    B, S, Hq, Hkv, D = 2, 19, 4, 2, 8
    q, k, v, do = rnd((B, S, Hq, D), 1), rnd((B, S, Hkv, D), 2), rnd((B, S, Hkv, D), 3), rnd((B, S, Hq, D), 4)
    bias = 1.5 * rnd(bshape, 5)
    mask = loop_mask(S, causal, *window)
    scale = 1 / math.sqrt(D)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = sdpa_biased(qt, kt, vt, bias, mask, scale)
    out.backward(do)
    o, m, l = dense.forward(q, k, v, causal=causal, window=window, bias=bias)
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12, rtol=0)
    dq, dk, dv = dense.backward(q, k, v, do, causal=causal, window=window, bias=bias)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11, rtol=0)


def test_row_constant_bias_changes_nothing_but_the_statistics():
    B, S, H, D = 1, 16, 2, 8
    q, k, v = rnd((B, S, H, D), 6), rnd((B, S, H, D), 7), rnd((B, S, H, D), 8)
    c = rnd((B, H, S, 1), 9)
    o, m, l = dense.forward(q, k, v, causal=True, bias=c)
    o0, m0, l0 = dense.forward(q, k, v, causal=True)
    np.testing.assert_allclose(o, o0, atol=1e-14, rtol=0)
    np.testing.assert_allclose(m, m0 + c.numpy()[..., 0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l, l0, rtol=1e-13, atol=0)


def test_minus_inf_bias_is_a_mask():
    """A key-padding bias (-inf on the last 5 keys) equals shortening the key sequence;
    a row whose keys are all removed gets o = 0, m = -inf, l = 0."""
    B, S, H, D = 2, 16, 2, 8
    q, k, v = rnd((B, S, H, D), 10), rnd((B, S, H, D), 11), rnd((B, S, H, D), 12)
    bias = torch.zeros((B, 1, 1, S), dtype=torch.float64)
    bias[..., S - 5:] = float("-inf")
    o, m, l = dense.forward(q, k, v, causal=False, bias=bias)
    o2, m2, l2 = dense.forward(q, k[:, :S - 5], v[:, :S - 5], causal=False)
    np.testing.assert_allclose(o, o2, atol=1e-14, rtol=0)
    bias2 = torch.zeros((1, 1, S, S), dtype=torch.float64)
    bias2[0, 0, 3, :] = float("-inf")
    o3, m3, l3 = dense.forward(q, k, v, causal=True, bias=bias2)
    assert np.all(o3[:, 3] == 0) and np.all(np.isneginf(m3[:, :, 3])) and np.all(l3[:, :, 3] == 0)
