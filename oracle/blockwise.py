"""The pages' blockwise recurrence and its ring schedule, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the method as "bpt.py" states it, in its own notation, used to pin that the
carried statistics reach the plain definition of ``oracle.dense``:

  * ``_blockwise_attention_fwd``: the queries are cut into chunks of
    ``query_chunk``, the keys into chunks of ``key_chunk``.  For every query chunk a
    carry (numerator [B, c, H, D], denominator [B, H, c], max_score [B, H, c]) is
    threaded through the key chunks.  For each visited key chunk:
        attn_weights = q_chunk k_chunk^T * scale (+ mask)
        max_score'   = max(max_score, rowmax(attn_weights))
        exp_weights  = exp(attn_weights - max_score')
        correction   = exp(max_score - max_score')
        numerator    = numerator * correction + exp_weights v_chunk
        denominator  = denominator * correction + rowsum(exp_weights)
    A chunk pair with no visible (query, key) pair is skipped (the causal
    ``skip_upper_half``; generalised here to any mask by positions).
  * ``_ring_attention_fwd``: the sequence is split into N equal blocks, one per ring
    member.  Member i keeps query block i; at ring step idx it holds kv block
    (i - idx) mod N (blocks travel one hop per step), and runs the blockwise pass
    over it with global chunk offsets.  After N steps: output = numerator /
    denominator.  The carry starts at numerator = 0, denominator = 0,
    max_score = -inf.

Masked entries are excluded exactly (-inf) and guarded so that a row with nothing
visible so far keeps a zero carry; this is the pages' result for every row that has
at least one visible key.
"""
from __future__ import annotations

import math

import numpy as np

from .dense import as_f64, kv_head_of, visible


def correction_factor(prev_max: np.ndarray, new_max_ref: np.ndarray) -> np.ndarray:
    """exp(max_score - max_score'): rescales the carried numerator and denominator."""
    return np.exp(prev_max - new_max_ref)


def init_carry(B: int, Sq: int, H: int, D: int):
    """(numerator, denominator, max_score) at the start of the ring."""
    return (np.zeros((B, Sq, H, D)), np.zeros((B, H, Sq)), np.full((B, H, Sq), -np.inf))


def blockwise_pass(q, k, v, carry, *, q_pos0: int, kv_pos0: int, query_chunk: int,
                   key_chunk: int, causal: bool, window=(-1, -1), scale=None):
    """One blockwise pass of a query block over one kv block, updating the carry.

    q [B, Sq, Hq, D]; k [B, Skv, Hkv, D]; v [B, Skv, Hkv, Dv]; carry as ``init_carry``
    (numerator with Dv columns).  Returns the new
    carry (numerator, denominator, max_score).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)
    assert Sq % query_chunk == 0 and Skv % key_chunk == 0
    numerator, denominator, max_score = (np.array(c, dtype=np.float64) for c in carry)
    wl, wr = window
    for qc in range(Sq // query_chunk):
        qs = slice(qc * query_chunk, (qc + 1) * query_chunk)
        q_positions = q_pos0 + np.arange(qc * query_chunk, (qc + 1) * query_chunk)
        for kc in range(Skv // key_chunk):
            ks = slice(kc * key_chunk, (kc + 1) * key_chunk)
            k_positions = kv_pos0 + np.arange(kc * key_chunk, (kc + 1) * key_chunk)
            mask = visible(q_positions, k_positions, causal, wl, wr)
            if not mask.any():
                continue                                   # skipped chunk pair
            for b in range(B):
                for h in range(Hq):
                    g = kv_head_of(h, G)
                    w = scale * (q[b, qs, h, :] @ k[b, ks, g, :].T)
                    w = np.where(mask, w, -np.inf)
                    prev = max_score[b, h, qs]
                    new = np.maximum(prev, w.max(axis=1))
                    ref = np.where(np.isfinite(new), new, 0.0)
                    exp_weights = np.exp(w - ref[:, None])
                    correction = correction_factor(prev, ref)
                    numerator[b, qs, h, :] = (numerator[b, qs, h, :] * correction[:, None]
                                              + exp_weights @ v[b, ks, g, :])
                    denominator[b, h, qs] = denominator[b, h, qs] * correction + exp_weights.sum(axis=1)
                    max_score[b, h, qs] = new
    return numerator, denominator, max_score


def finalize(carry):
    """output = numerator / denominator (rows with denominator 0 give 0)."""
    numerator, denominator, _ = carry
    den = np.transpose(denominator, (0, 2, 1))[..., None]       # [B, Sq, H, 1]
    return np.where(den > 0, numerator / np.where(den > 0, den, 1.0), 0.0)


def ring_forward(q, k, v, *, n_blocks: int, query_chunk: int, key_chunk: int, causal: bool,
                 window=(-1, -1), scale=None):
    """Ring schedule simulated on one host; returns (o, m, l) like ``dense.forward``."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, S, Hq, _ = q.shape
    Dv = v.shape[3]                                 # value head dim (may differ from q/k's)
    assert S % n_blocks == 0 and k.shape[1] == S
    blk = S // n_blocks
    o = np.zeros((B, S, Hq, Dv))
    m = np.zeros((B, Hq, S))
    l = np.zeros((B, Hq, S))
    for i in range(n_blocks):                       # ring member i holds query block i
        qi = slice(i * blk, (i + 1) * blk)
        carry = init_carry(B, blk, Hq, Dv)
        for idx in range(n_blocks):                 # ring step idx
            j = (i - idx) % n_blocks                # kv block held at this step
            kj = slice(j * blk, (j + 1) * blk)
            carry = blockwise_pass(q[:, qi], k[:, kj], v[:, kj], carry, q_pos0=i * blk,
                                   kv_pos0=j * blk, query_chunk=query_chunk,
                                   key_chunk=key_chunk, causal=causal, window=window,
                                   scale=scale)
        o[:, qi] = finalize(carry)
        l[:, :, qi] = carry[1]
        m[:, :, qi] = carry[2]
    return o, m, l
