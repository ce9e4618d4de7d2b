"""Pins of the dense oracle's analytic gradient.

* central finite differences of the forward (fp64, tiny shapes);
* torch autograd through fp64 scaled_dot_product_attention (an independent routine);
* closed forms / invariants: sum_j dK_j = 0 (softmax shift invariance),
  sum_j dV_j = sum over the group of sum_i dO_i, and with a window of 0 keys to the
  left dQ = dK = 0 and dV = the group's dO.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dense


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def loss(q, k, v, do, **kw):
    o, _, _ = dense.forward(q, k, v, **kw)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,window,qp0,kp0,Dv", [
    (True, (-1, -1), 0, 0, 4), (True, (3, 0), 0, 0, 4), (False, (2, 1), 0, 0, 4), (True, (-1, -1), 4, 0, 4),
    (True, (-1, -1), 0, 0, 2), (False, (2, 1), 3, 0, 6)])
def test_finite_differences(causal, window, qp0, kp0, Dv):
    """Dv != D covers a value head dim of its own (the MLA case)."""
    B, Sq, Skv, Hq, Hkv, D = 1, 9, 11, 2, 1, 4
    q, k, v, do = (rnd((B, Sq, Hq, D), 1).numpy(), rnd((B, Skv, Hkv, D), 2).numpy(),
                   rnd((B, Skv, Hkv, Dv), 3).numpy(), rnd((B, Sq, Hq, Dv), 4).numpy())
    kw = dict(causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0)
    dq, dk, dv = dense.backward(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v, do, **kw)
            x[idx] = old - h
            lm = loss(q, k, v, do, **kw)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("Hq,Hkv,causal,window,Dv", [(4, 2, True, (-1, -1), 8), (6, 3, True, (5, 0), 8),
                                                       (2, 2, False, (-1, -1), 8), (8, 2, True, (-1, -1), 4),
                                                       (4, 1, True, (7, 0), 4)])
def test_matches_torch_autograd(Hq, Hkv, causal, window, Dv):
    B, S, D = 2, 23, 8
    q, k, v, do = rnd((B, S, Hq, D), 5), rnd((B, S, Hkv, D), 6), rnd((B, S, Hkv, Dv), 7), rnd((B, S, Hq, Dv), 8)
    mask = np.zeros((S, S), dtype=bool)
    for i in range(S):
        for j in range(S):
            ok = (not causal or j <= i) and (window[1] < 0 or j <= i + window[1]) and \
                 (window[0] < 0 or j >= i - window[0])
            mask[i, j] = ok
    Q, K, V = (t.clone().permute(0, 2, 1, 3).requires_grad_(True) for t in (q, k, v))
    G = Hq // Hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K.repeat_interleave(G, 1), V.repeat_interleave(G, 1), attn_mask=torch.from_numpy(mask))
    out.backward(do.permute(0, 2, 1, 3))
    dq, dk, dv = dense.backward(q, k, v, do, causal=causal, window=window)
    np.testing.assert_allclose(dq, Q.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, K.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, V.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)


def test_gradient_sums():
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 8
    q, k, v, do = rnd((B, S, Hq, D), 9), rnd((B, S, Hkv, D), 10), rnd((B, S, Hkv, D), 11), rnd((B, S, Hq, D), 12)
    dq, dk, dv = dense.backward(q, k, v, do, causal=True, window=(9, 0))
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12, rtol=0)
    G = Hq // Hkv
    do_group = do.numpy().reshape(B, S, Hkv, G, D).sum(axis=3)
    np.testing.assert_allclose(dv.sum(axis=1), do_group.sum(axis=1), atol=1e-12, rtol=0)


def test_zero_left_window_gradients():
    B, S, Hq, Hkv, D = 1, 17, 4, 2, 8
    q, k, v, do = rnd((B, S, Hq, D), 13), rnd((B, S, Hkv, D), 14), rnd((B, S, Hkv, D), 15), rnd((B, S, Hq, D), 16)
    dq, dk, dv = dense.backward(q, k, v, do, causal=True, window=(0, 0))
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    G = Hq // Hkv
    np.testing.assert_allclose(dv, do.numpy().reshape(B, S, Hkv, G, D).sum(axis=3), atol=1e-14, rtol=0)


def test_scale_enters_dq_and_dk_linearly():
    """With scale c on the logits, d/dq of sum(dO*O) carries c (chain rule): compare a
    scale-c run on q with a scale-1 run on c*q."""
    B, S, H, D = 1, 12, 2, 4
    q, k, v, do = rnd((B, S, H, D), 17), rnd((B, S, H, D), 18), rnd((B, S, H, D), 19), rnd((B, S, H, D), 20)
    c = 0.37
    dq_a, dk_a, dv_a = dense.backward(q, k, v, do, causal=True, scale=c)
    dq_b, dk_b, dv_b = dense.backward(q * c, k, v, do, causal=True, scale=1.0)
    np.testing.assert_allclose(dq_a, c * dq_b, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dk_a, dk_b, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dv_a, dv_b, atol=1e-13, rtol=0)
    assert math.isfinite(float(np.abs(dq_a).max()))
