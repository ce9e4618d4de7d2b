"""Attention over gathered candidate keys (window ++ selected blocks), fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``faiss_block_attention`` of the "AnnAttention" page ("Core code"):
  * heads are flattened into one joint embedding E = H * D per token;
  * every token t attends to a candidate list made of
      - a sliding window of ``window`` keys ending at t (inclusive), padded with
        zero vectors before the start of the sequence, then
      - for each of its selected block indices (in the stored ascending order) the
        ``block_size`` rows of that block; an index of -1 is clamped to token 0 for
        every row, as the page clamps negative item indices to 0;
    duplicates are kept;
  * logits = q_t . k_slot / sqrt(E); softmax over all slots with no mask (zero
    padding slots take part with logit 0 and value 0); o_t = sum p * v_slot.

The window helper and the block-to-item helper are not shown on the page; the
readings above (window ends at t inclusive, zero padding; block c -> rows c*bs ..
c*bs+bs-1) are pinned only to themselves -- parity unpinned against the originals.
A selected block whose rows run past the end of the key sequence is outside what the
page defines: its selection never returns one, and its gather would fail on it.  The
functions here raise ValueError for such an index.

Decoding (the page's inference mode trims the windows to the last position and attends
the new tokens against the whole key cache): ``q_pos0`` places the query rows at
positions q_pos0 .. q_pos0 + Sq - 1 of a key / value cache of Skv rows; every token's
slots are as above, taken from the cache.  The page's inference-mode loop is garbled in
the extracted text, so this reading is pinned only to itself (equality with the
full-sequence rows): parity unpinned against the page.
"""
from __future__ import annotations

import math

import numpy as np

from .dense import as_f64


def _flat(x):
    x = as_f64(x)
    if x.ndim == 4:
        x = x.reshape(x.shape[0], x.shape[1], -1)
    return x


def candidate_positions(t: int, sel_row, *, window: int, block_size: int, seqlen=None):
    """(positions, is_zero_pad) of token t's candidate slots, in list order.  With
    ``seqlen`` given, a selected block with rows at or past it raises ValueError (the
    page's gather of item indices is only defined inside the sequence)."""
    pos, pad = [], []
    for w in range(window):
        p = t - window + 1 + w
        pos.append(max(p, 0))
        pad.append(p < 0)
    for c in sel_row:
        c = int(c)
        if seqlen is not None and c >= 0 and (c + 1) * block_size > seqlen:
            raise ValueError(f"selected block {c} has rows past the end of the {seqlen}-row key sequence")
        for r in range(block_size):
            p = c * block_size + r
            pos.append(0 if p < 0 else p)
            pad.append(False)
    return np.asarray(pos, dtype=np.int64), np.asarray(pad, dtype=bool)


def sparse_attention(q, k, v, sel, *, window: int, block_size: int, scale=None, tokens=None,
                     q_pos0: int = 0):
    """o [B, Sq, E], m [B, Sq], l [B, Sq] in fp64 (m, l: max logit and sum of exp(logit - m))
    for query rows at positions q_pos0 + i of the key / value sequence (length Skv).

    ``tokens`` restricts the evaluation to sampled query rows (others are NaN).
    """
    q, k, v = _flat(q), _flat(k), _flat(v)
    sel = np.asarray(sel.cpu() if hasattr(sel, "cpu") else sel)
    B, S, E = q.shape
    Skv = k.shape[1]
    sc = 1.0 / math.sqrt(E) if (scale is None or scale <= 0) else float(scale)
    fill = np.nan if tokens is not None else 0.0
    o = np.full((B, S, E), fill)
    m = np.full((B, S), fill)
    l = np.full((B, S), fill)
    toks = range(S) if tokens is None else tokens
    for b in range(B):
        for t in toks:
            pos, pad = candidate_positions(q_pos0 + t, sel[b, t], window=window, block_size=block_size,
                                           seqlen=Skv)
            K = np.where(pad[:, None], 0.0, k[b, pos])
            V = np.where(pad[:, None], 0.0, v[b, pos])
            s = sc * (K @ q[b, t])
            mt = s.max()
            p = np.exp(s - mt)
            lt = p.sum()
            o[b, t] = (p @ V) / lt
            m[b, t] = mt
            l[b, t] = lt
    return o, m, l


def sparse_attention_backward(q, k, v, sel, do, *, window: int, block_size: int, scale=None):
    """Gradient of ``sparse_attention`` contracted with dO: (dq, dk, dv), each [B, S, E] fp64.

    Per token t, with its candidate slots j (keys K_j, values V_j; zero pads are
    constants): P = softmax(s), D_t = dO_t . O_t, dP_j = dO_t . V_j,
    dS_j = P_j (dP_j - D_t), dq_t = scale sum_j dS_j K_j, and every slot that reads
    a sequence row p passes dk_p += scale dS_j q_t, dv_p += P_j dO_t back to it (a
    row read by several slots -- duplicates, the -1 clamp to token 0 -- collects all of
    them; zero pads collect nothing).
    """
    q, k, v, do = _flat(q), _flat(k), _flat(v), _flat(do)
    sel = np.asarray(sel.cpu() if hasattr(sel, "cpu") else sel)
    B, S, E = q.shape
    sc = 1.0 / math.sqrt(E) if (scale is None or scale <= 0) else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for t in range(S):
            pos, pad = candidate_positions(t, sel[b, t], window=window, block_size=block_size, seqlen=S)
            K = np.where(pad[:, None], 0.0, k[b, pos])
            V = np.where(pad[:, None], 0.0, v[b, pos])
            s = sc * (K @ q[b, t])
            p = np.exp(s - s.max())
            P = p / p.sum()
            O = P @ V
            Dt = do[b, t] @ O
            dP = V @ do[b, t]
            dS = P * (dP - Dt)
            dq[b, t] = sc * (dS @ K)
            live = ~pad
            np.add.at(dk[b], pos[live], sc * dS[live, None] * q[b, t][None, :])
            np.add.at(dv[b], pos[live], P[live, None] * do[b, t][None, :])
    return dq, dk, dv
