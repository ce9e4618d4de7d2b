"""Pins: the pages' blockwise carry, run in ring order, reaches the plain definition.

This pins both directions at once: ``oracle.blockwise`` is the recurrence as the
pages state it, ``oracle.dense`` is the definition pinned to torch's SDPA elsewhere.
It also pins the step contract used by the library's carry-in / no-finalize flags:
running the ring in two halves with the carry handed over equals one run.
"""
import numpy as np
import pytest
import torch

from oracle import blockwise, dense


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


@pytest.mark.parametrize("n_blocks,qc,kc,causal,window,Dv", [
    (4, 8, 8, True, (-1, -1), 8),
    (4, 4, 16, True, (-1, -1), 8),    # query and key chunks of different sizes
    (2, 16, 8, False, (-1, -1), 8),
    (8, 4, 4, True, (5, 0), 8),
    (1, 32, 32, True, (-1, -1), 8),   # one block: plain blockwise attention
    (4, 8, 8, True, (-1, -1), 4),     # value head dim of its own (MLA)
])
def test_ring_carry_equals_definition(n_blocks, qc, kc, causal, window, Dv):
    B, S, Hq, Hkv, D = 2, 64, 4, 2, 8
    q, k, v = rnd((B, S, Hq, D), 1), rnd((B, S, Hkv, D), 2), rnd((B, S, Hkv, Dv), 3)
    o_r, m_r, l_r = blockwise.ring_forward(q, k, v, n_blocks=n_blocks, query_chunk=qc,
                                           key_chunk=kc, causal=causal, window=window)
    o_d, m_d, l_d = dense.forward(q, k, v, causal=causal, window=window)
    np.testing.assert_allclose(o_r, o_d, atol=1e-12, rtol=0)
    np.testing.assert_allclose(m_r, m_d, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l_r, l_d, rtol=1e-12, atol=0)


def test_carry_handover_equals_single_pass():
    """Two passes over two kv halves with the carry handed over == one pass over all."""
    B, S, H, D = 1, 32, 2, 8
    q, k, v = rnd((B, S, H, D), 4), rnd((B, S, H, D), 5), rnd((B, S, H, D), 6)
    kw = dict(q_pos0=0, query_chunk=8, key_chunk=8, causal=True)
    c0 = blockwise.init_carry(B, S, H, D)
    one = blockwise.blockwise_pass(q, k, v, c0, kv_pos0=0, **kw)
    half = blockwise.blockwise_pass(q, k[:, 16:], v[:, 16:], c0, kv_pos0=16, **kw)
    two = blockwise.blockwise_pass(q, k[:, :16], v[:, :16], half, kv_pos0=0, **kw)
    np.testing.assert_allclose(blockwise.finalize(one), blockwise.finalize(two), atol=1e-13, rtol=0)
    o_d, _, _ = dense.forward(q, k, v, causal=True)
    np.testing.assert_allclose(blockwise.finalize(two), o_d, atol=1e-13, rtol=0)


def test_skipped_chunks_are_exactly_the_invisible_ones():
    """A pass over a kv block entirely in the future leaves the carry unchanged."""
    B, S, H, D = 1, 16, 1, 4
    q, k, v = rnd((B, S, H, D), 7), rnd((B, S, H, D), 8), rnd((B, S, H, D), 9)
    c0 = blockwise.init_carry(B, S, H, D)
    c1 = blockwise.blockwise_pass(q, k, v, c0, q_pos0=0, kv_pos0=16, query_chunk=4, key_chunk=4,
                                  causal=True)
    for a, b in zip(c0, c1):
        np.testing.assert_array_equal(a, b)
