"""Pins of the oracle's sink softmax (the TransformerEngine page, "Other attention knobs":
``softmax_type="off_by_one"`` / ``"learnable"``).

* an independent library routine: torch fp64 scaled_dot_product_attention over the keys
  plus one extra key whose value vector is zero and whose logit is set to z by an
  additive float mask -- the "extra key" reading of a sink, built with torch ops only;
* torch autograd through that routine for dq, dk, dv and the sink logits;
* central finite differences of the sink gradient;
* closed forms: a window of 0 keys to the left gives O_i = v_i / (1 + exp(z - s_ii));
  z -> -inf gives the plain softmax; the statistics m, l ignore the sink.
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


def sdpa_with_sink_key(q, k, v, z, mask, scale):
    """SDPA over [keys, one zero key] with the zero key's logit forced to z_h."""
    B, S, Hq, D = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    G = Hq // Hkv
    Q = q.permute(0, 2, 1, 3)
    K = torch.cat([k.permute(0, 2, 1, 3).repeat_interleave(G, 1), torch.zeros(B, Hq, 1, D, dtype=q.dtype)], 2)
    V = torch.cat([v.permute(0, 2, 1, 3).repeat_interleave(G, 1), torch.zeros(B, Hq, 1, Dv, dtype=q.dtype)], 2)
    bias = torch.zeros(B, Hq, S, S + 1, dtype=q.dtype)
    bias[..., :S] = torch.where(torch.from_numpy(mask), 0.0, float("-inf"))
    bias = bias + torch.cat([torch.zeros(B, Hq, S, S, dtype=q.dtype),
                             z.view(1, Hq, 1, 1).expand(B, Hq, S, 1)], 3)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=bias, scale=scale)
    return out.permute(0, 2, 1, 3)


@pytest.mark.parametrize("causal,window,G,Dv", [(True, (-1, -1), 2, 8), (True, (5, 0), 4, 8),
                                                (False, (-1, 3), 1, 4), (True, (-1, -1), 2, 4)])
def test_sink_forward_and_backward_match_torch(causal, window, G, Dv):
    B, S, Hkv, D = 2, 21, 2, 8
    Hq = Hkv * G
    q, k, v, do = rnd((B, S, Hq, D), 1), rnd((B, S, Hkv, D), 2), rnd((B, S, Hkv, Dv), 3), rnd((B, S, Hq, Dv), 4)
    z = rnd((Hq,), 5)
    mask = loop_mask(S, causal, *window)
    scale = 1 / math.sqrt(D)
    qt, kt, vt, zt = (t.clone().requires_grad_(True) for t in (q, k, v, z))
    out = sdpa_with_sink_key(qt, kt, vt, zt, mask, scale)
    out.backward(do)
    o, m, l = dense.forward(q, k, v, causal=causal, window=window, sink=z)
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12, rtol=0)
    o_plain, m_plain, l_plain = dense.forward(q, k, v, causal=causal, window=window)
    np.testing.assert_array_equal(m, m_plain)             # statistics of the keys alone
    np.testing.assert_array_equal(l, l_plain)
    dq, dk, dv, dz = dense.backward(q, k, v, do, causal=causal, window=window, sink=z)
    for name, a, b in (("dq", dq, qt.grad), ("dk", dk, kt.grad), ("dv", dv, vt.grad), ("dz", dz, zt.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-11, rtol=0, err_msg=name)


def test_off_by_one_is_a_zero_sink():
    """softmax_1: 1 + sum exp in the denominator, i.e. an extra key with logit 0."""
    B, S, H, D = 1, 12, 2, 4
    q, k, v = rnd((B, S, H, D), 6), rnd((B, S, H, D), 7), rnd((B, S, H, D), 8)
    o, m, l = dense.forward(q, k, v, causal=True, sink=np.zeros(H))
    s = np.einsum("bihd,bjhd->bhij", q.numpy(), k.numpy()) / math.sqrt(D)
    s = np.where(np.tril(np.ones((S, S), dtype=bool)), s, -np.inf)
    e = np.exp(s)                                          # small logits: no shift needed
    ref = np.einsum("bhij,bjhd->bihd", e / (1.0 + e.sum(-1, keepdims=True)), v.numpy())
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_sink_with_zero_left_window_closed_form():
    """Each row sees only its own key: O_i = v_i * e^{s_ii} / (e^{s_ii} + e^{z})."""
    B, S, H, D = 1, 10, 3, 4
    q, k, v = rnd((B, S, H, D), 9), rnd((B, S, H, D), 10), rnd((B, S, H, D), 11)
    z = np.array([0.3, -2.0, 1.5])
    o, _, _ = dense.forward(q, k, v, causal=True, window=(0, 0), sink=z)
    s = (q.numpy() * k.numpy()).sum(-1) / math.sqrt(D)          # [B, S, H]
    w = 1.0 / (1.0 + np.exp(z[None, None, :] - s))
    np.testing.assert_allclose(o, v.numpy() * w[..., None], atol=1e-13, rtol=0)


def test_very_negative_sink_is_plain_softmax():
    B, S, H, D = 1, 14, 2, 8
    q, k, v = rnd((B, S, H, D), 12), rnd((B, S, H, D), 13), rnd((B, S, H, D), 14)
    o, _, _ = dense.forward(q, k, v, causal=True, sink=np.full(H, -800.0))
    o0, _, _ = dense.forward(q, k, v, causal=True)
    np.testing.assert_allclose(o, o0, atol=1e-15, rtol=0)


def test_sink_gradient_finite_differences():
    B, S, Hq, Hkv, D = 1, 9, 2, 1, 4
    q, k, v, do = (rnd((B, S, Hq, D), 15).numpy(), rnd((B, S, Hkv, D), 16).numpy(),
                   rnd((B, S, Hkv, D), 17).numpy(), rnd((B, S, Hq, D), 18).numpy())
    z = np.array([0.4, -0.7])
    _, _, _, dz = dense.backward(q, k, v, do, causal=True, sink=z)
    h = 1e-6
    for i in range(Hq):
        zp, zm = z.copy(), z.copy()
        zp[i] += h
        zm[i] -= h
        lp = float((dense.forward(q, k, v, causal=True, sink=zp)[0] * do).sum())
        lm = float((dense.forward(q, k, v, causal=True, sink=zm)[0] * do).sum())
        assert abs((lp - lm) / (2 * h) - dz[i]) < 1e-7
