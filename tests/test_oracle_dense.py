"""Pins of the dense oracle's forward against things other than itself.

* an independent library routine: torch CPU fp64 scaled_dot_product_attention with a
  boolean mask built here by explicit loops over (i, j);
* closed forms (window of 0 keys to the left, zero queries, constant values);
* invariants (rows of P sum to 1, GQA equals MHA on repeated K/V, a window wider
  than the sequence equals causal, shifting both position origins changes nothing);
* a hand-worked example stored under tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale)


def loop_mask(Sq, Skv, causal, wl, wr, q_pos0=0, kv_pos0=0):
    """Visibility by explicit loops (written independently of the oracle)."""
    M = np.zeros((Sq, Skv), dtype=bool)
    for i in range(Sq):
        for j in range(Skv):
            qp, kp = q_pos0 + i, kv_pos0 + j
            ok = True
            if causal and kp > qp:
                ok = False
            if wr >= 0 and kp > qp + wr:
                ok = False
            if wl >= 0 and kp < qp - wl:
                ok = False
            M[i, j] = ok
    return M


def sdpa_reference(q, k, v, mask, scale):
    """torch fp64 SDPA; q [B,S,Hq,D] -> BHSD with GQA expansion done by torch."""
    Q = q.permute(0, 2, 1, 3)
    K = k.permute(0, 2, 1, 3)
    V = v.permute(0, 2, 1, 3)
    G = Q.shape[1] // K.shape[1]
    K = K.repeat_interleave(G, dim=1)
    V = V.repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(mask), scale=scale)
    s = (Q @ K.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    return out.permute(0, 2, 1, 3).numpy(), s.amax(-1).numpy(), torch.logsumexp(s, -1).numpy()


CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal, window, q_pos0, kv_pos0
    (2, 37, 37, 4, 2, 8, True, (-1, -1), 0, 0),
    (1, 64, 64, 4, 4, 16, False, (-1, -1), 0, 0),
    (2, 50, 50, 6, 2, 8, True, (7, 0), 0, 0),
    (1, 40, 40, 2, 1, 8, False, (5, 3), 0, 0),
    (1, 32, 48, 4, 2, 8, True, (-1, -1), 16, 0),       # queries after the keys start
    (1, 24, 24, 2, 2, 4, True, (3, -1), 100, 98),      # shifted origins, window
    (1, 20, 30, 3, 1, 8, False, (-1, 2), 10, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_matches_torch_sdpa(case):
    B, Sq, Skv, Hq, Hkv, D, causal, window, qp0, kp0 = case
    q, k, v = rnd((B, Sq, Hq, D), 1), rnd((B, Skv, Hkv, D), 2), rnd((B, Skv, Hkv, D), 3)
    scale = 0.7 / math.sqrt(D)
    mask = loop_mask(Sq, Skv, causal, *window, qp0, kp0)
    assert mask.any(axis=1).all(), "every row must see a key for the SDPA comparison"
    o_ref, m_ref, lse_ref = sdpa_reference(q, k, v, mask, scale)
    o, m, l = dense.forward(q, k, v, causal=causal, window=window, scale=scale,
                            q_pos0=qp0, kv_pos0=kp0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, m_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m + np.log(l), lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window,G", [(True, (-1, -1), 2), (True, (6, 0), 4), (False, (-1, 3), 1)])
def test_value_head_dim_differs_matches_torch_sdpa(causal, window, G):
    """v (and so o) with its own head dim (the TransformerEngine page's DeepSeek-style
    MLA case, section 4); torch's SDPA accepts Ev != E."""
    B, S, Hkv, D, Dv = 2, 33, 2, 16, 8
    q, k, v = rnd((B, S, Hkv * G, D), 21), rnd((B, S, Hkv, D), 22), rnd((B, S, Hkv, Dv), 23)
    mask = loop_mask(S, S, causal, *window)
    assert mask.any(axis=1).all()
    scale = 1 / math.sqrt(D)                       # the q/k head dim, not Dv
    o_ref, m_ref, lse_ref = sdpa_reference(q, k, v, mask, scale)
    o, m, l = dense.forward(q, k, v, causal=causal, window=window)
    assert o.shape == (B, S, Hkv * G, Dv)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, m_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m + np.log(l), lse_ref, rtol=0, atol=1e-12)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = rnd((1, 16, 2, 8), 4), rnd((1, 16, 2, 8), 5), rnd((1, 16, 2, 8), 6)
    mask = loop_mask(16, 16, True, -1, -1)
    o_ref, _, _ = sdpa_reference(q, k, v, mask, 1 / math.sqrt(8))
    o, _, _ = dense.forward(q, k, v, causal=True)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)


def test_window_zero_left_returns_own_value():
    """left = 0 with causal: each query sees only its own key -> O = v_i, l = 1, m = s_ii."""
    B, S, Hq, Hkv, D = 2, 33, 4, 2, 8
    q, k, v = rnd((B, S, Hq, D), 7), rnd((B, S, Hkv, D), 8), rnd((B, S, Hkv, D), 9)
    o, m, l = dense.forward(q, k, v, causal=True, window=(0, 0))
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(o[:, :, h], v[:, :, h // G].numpy(), atol=1e-14, rtol=0)
        sii = (q[:, :, h] * k[:, :, h // G]).sum(-1).numpy() / math.sqrt(D)
        np.testing.assert_allclose(m[:, h], sii, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l, 1.0, atol=0, rtol=0)


def test_zero_queries_average_visible_values():
    """q = 0: all logits are 0 -> O = mean of visible V, m = 0, l = number visible."""
    B, S, Hq, Hkv, D = 1, 40, 2, 1, 8
    q = torch.zeros((B, S, Hq, D), dtype=torch.float64)
    k, v = rnd((B, S, Hkv, D), 10), rnd((B, S, Hkv, D), 11)
    window = (5, 0)
    o, m, l = dense.forward(q, k, v, causal=True, window=window)
    for i in range(S):
        lo = max(0, i - 5)
        np.testing.assert_allclose(o[0, i, 0], v[0, lo:i + 1, 0].numpy().mean(0), atol=1e-14, rtol=0)
        assert l[0, 0, i] == i - lo + 1
    assert np.all(m == 0)


def test_constant_values_return_the_constant():
    B, S, Hq, Hkv, D = 1, 30, 4, 2, 8
    q, k = rnd((B, S, Hq, D), 12), rnd((B, S, Hkv, D), 13)
    c = rnd((D,), 14)
    v = c.expand(B, S, Hkv, D).clone()
    o, _, _ = dense.forward(q, k, v, causal=True, window=(9, 0))
    np.testing.assert_allclose(o, np.broadcast_to(c.numpy(), o.shape), atol=1e-13, rtol=0)


def test_probability_rows_sum_to_one_and_respect_mask():
    B, S, Hq, Hkv, D = 1, 25, 2, 1, 4
    q, k = rnd((B, S, Hq, D), 15), rnd((B, S, Hkv, D), 16)
    P = dense.probs(q, k, causal=True, window=(6, 0))
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14, rtol=0)
    mask = loop_mask(S, S, True, 6, 0)
    assert np.all(P[..., ~mask] == 0)
    assert np.all(P[..., mask] > 0)


def test_gqa_equals_mha_on_repeated_kv():
    B, S, Hq, Hkv, D = 2, 20, 6, 2, 8
    q, k, v = rnd((B, S, Hq, D), 17), rnd((B, S, Hkv, D), 18), rnd((B, S, Hkv, D), 19)
    o_g, m_g, l_g = dense.forward(q, k, v, causal=True)
    G = Hq // Hkv
    k_r, v_r = k.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2)
    o_m, m_m, l_m = dense.forward(q, k_r, v_r, causal=True)
    np.testing.assert_array_equal(o_g, o_m)
    np.testing.assert_array_equal(m_g, m_m)
    np.testing.assert_array_equal(l_g, l_m)


def test_wide_window_equals_causal():
    B, S, H, D = 1, 31, 2, 8
    q, k, v = rnd((B, S, H, D), 20), rnd((B, S, H, D), 21), rnd((B, S, H, D), 22)
    a = dense.forward(q, k, v, causal=True)
    b = dense.forward(q, k, v, causal=True, window=(S - 1, 0))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_shift_invariance_of_positions():
    B, S, H, D = 1, 28, 2, 8
    q, k, v = rnd((B, S, H, D), 23), rnd((B, S, H, D), 24), rnd((B, S, H, D), 25)
    a = dense.forward(q, k, v, causal=True, window=(4, 0))
    b = dense.forward(q, k, v, causal=True, window=(4, 0), q_pos0=5000, kv_pos0=5000)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_sampled_rows_equal_full_rows():
    B, S, Hq, Hkv, D = 1, 300, 4, 2, 8
    q, k, v = rnd((B, S, Hq, D), 26), rnd((B, S, Hkv, D), 27), rnd((B, S, Hkv, D), 28)
    full = dense.forward(q, k, v, causal=True)
    rows = np.array([0, 1, 77, 255, 256, 299])
    samp = dense.forward(q, k, v, causal=True, rows=rows, heads=[1, 3])
    for f, s_ in zip(full, samp):
        if f.ndim == 4:
            np.testing.assert_array_equal(f[:, rows][:, :, [1, 3]], s_[:, rows][:, :, [1, 3]])
        else:
            np.testing.assert_array_equal(f[:, [1, 3]][:, :, rows], s_[:, [1, 3]][:, :, rows])


def test_row_without_visible_key():
    """Queries before every key position: O = 0, m = -inf, l = 0."""
    q, k, v = rnd((1, 4, 1, 4), 29), rnd((1, 4, 1, 4), 30), rnd((1, 4, 1, 4), 31)
    o, m, l = dense.forward(q, k, v, causal=True, q_pos0=0, kv_pos0=2)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(m[0, 0, :2])) and np.all(l[0, 0, :2] == 0)
    assert np.all(np.isfinite(m[0, 0, 2:]))


def test_visible_pair_count_matches_mask():
    for (S, causal, w) in [(64, True, (-1, -1)), (64, True, (5, 0)), (50, False, (3, 2))]:
        assert dense.visible_pairs(S, S, causal=causal, window=w) == loop_mask(S, S, causal, *w).sum()


def test_hand_worked_example():
    """A 2-query, 2-key example whose softmax weights were derived by hand."""
    with open(os.path.join(GOLDEN, "hand_worked_attention.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.array(g["k"], dtype=np.float64)[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    o, m, l = dense.forward(q, k, v, causal=g["causal"], scale=g["scale"])
    np.testing.assert_allclose(o[0, :, 0], np.array(g["o"]), atol=1e-15, rtol=0)
    np.testing.assert_allclose(m[0, 0], np.array(g["m"]), atol=1e-15, rtol=0)
    np.testing.assert_allclose(l[0, 0], np.array(g["l"]), atol=1e-15, rtol=0)
