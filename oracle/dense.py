"""Dense exact softmax attention from its definition, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product.

Definition followed (one (batch, q head) pair at a time):
  * q head h reads kv head floor(h / G), G = Hq / Hkv -- the GQA mapping of
    "JAX: Single-GPU Attention with TransformerEngine", section 1, ``_repeat_kv_for_gqa``
    (each kv head is repeated G times along the head axis, so consecutive q heads
    share one kv head).
  * positions are global: query row i sits at q_pos0 + i, key row j at kv_pos0 + j,
    as the chunk offsets of "bpt.py" (``_ring_attention_fwd`` computes chunk start
    indices from the block index; ``_chunk_attention_bias`` turns them into offsets).
  * a pair is visible iff (causal => key <= query) and (right >= 0 => key <= query +
    right) and (left >= 0 => key >= query - left); -1 means unbounded.  The causal
    rule is ``_chunk_attention_bias`` of "bpt.py"; the window rule is
    ``_make_causal_swa_mask`` of the TransformerEngine page, section 1 (both window
    ends inclusive).
  * s_ij = scale * q_i . k_j with scale = 1/sqrt(D) unless given ("bpt.py" divides
    logits by sqrt(d); the TransformerEngine page multiplies by d^-1/2 and lets
    ``scale_factor`` override it, "Other attention knobs").
  * invisible pairs are excluded exactly (the pages add the most negative finite
    number; for any row with at least one visible key this is the same result).
  * m_i = max over visible s_ij, l_i = sum over visible exp(s_ij - m_i),
    P_ij = exp(s_ij - m_i) / l_i, O_i = sum_j P_ij v_j.
  * a row with no visible key gets O = 0, m = -inf, l = 0.

Backward (analytic gradient of the same function; the einsum comments and the
blockwise body of ``_blockwise_attention_bwd`` in "bpt.py"):
  D_i = dO_i . O_i,  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i),
  dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
with dK and dV summed over the G q heads that share a kv head (the gradient of the
repeat in the GQA mapping).

Additive bias ("bpt.py": ``ring_attention`` / ``blockwise_attn`` take a bias that
broadcasts to (batch, heads, q_len, kv_len) and is added to the scaled logits of each
chunk, ``_chunk_attention_bias``; the page returns no gradient for it): s_ij gains
bias[b, h, i, j] (natural units) before the mask and the softmax.  A bias of -inf removes
a pair like the mask does.

Dropout ("bpt.py": ``_blockwise_attention_fwd`` / ``_blockwise_attention_bwd`` draw a
Bernoulli(attn_pdrop) array over (batch, heads, q_len, kv_len) and
``_chunk_attention_bias`` adds it times the dtype's most negative value to the logits):
a dropped pair leaves the softmax like a masked one, and the other weights are not
rescaled.  The array is an input here (the page draws it from a JAX key; any source of
the same Bernoulli draws will do), True = dropped, broadcastable like the bias.

Sink softmax ("JAX: Single-GPU Attention with TransformerEngine", "Other attention
knobs": ``softmax_type="off_by_one"`` or ``"learnable"``; the page names the options only,
so this is the plain reading of their names): every row's softmax gets one more term in
its denominator, exp(z_h) for a per-q-head sink logit z_h in the units of the scaled
logits, with nothing added to the numerator -- as if each row also saw one extra key
with logit z_h and a zero value vector.  "off_by_one" is z_h = 0 (the 1 + sum exp form);
"learnable" takes z_h as an input and has a gradient:
  P_ij = exp(s_ij) / (exp(z_h) + sum_k exp(s_ik)),  P_sink,i = exp(z_h) / (same),
  dS_ij = P_ij (dP_ij - D_i) as before, and dz_h = -sum_{b,i} P_sink,i D_i.
The statistics m, l stay those of the keys alone (the sink enters only when the output
is normalised), so the blockwise carry is unchanged.

The value head dim Dv may differ from the q/k head dim D (the DeepSeek-style MLA case
of the TransformerEngine page, section 4: q/k 128, v 64); nothing above needs them
equal: O, dO and dV have Dv columns, Q, K, dQ and dK have D, and the default scale
stays 1/sqrt(D).

Rows are processed in slices only to bound memory; every row's softmax is computed
over that row's complete visible key range, so this is the plain definition.
"""
from __future__ import annotations

import math

import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp32) or array to an fp64 numpy array."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(hq: int, group: int) -> int:
    """GQA mapping: q head hq reads kv head hq // G (repeat, not modulo)."""
    return hq // group


def visible(q_pos, k_pos, causal: bool, window_left: int = -1, window_right: int = -1) -> np.ndarray:
    """Boolean [len(q_pos), len(k_pos)]: which (query, key) pairs may attend."""
    qp = np.asarray(q_pos, dtype=np.int64)[:, None]
    kp = np.asarray(k_pos, dtype=np.int64)[None, :]
    ok = np.ones((qp.shape[0], kp.shape[1]), dtype=bool)
    if causal:
        ok &= kp <= qp
    if window_right >= 0:
        ok &= kp <= qp + window_right
    if window_left >= 0:
        ok &= kp >= qp - window_left
    return ok


def scores(q_rows: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """s = scale * q k^T for [R, D] x [C, D] -> [R, C]."""
    return scale * (q_rows @ k_rows.T)


def grad_scores(P: np.ndarray, dP: np.ndarray, Di: np.ndarray) -> np.ndarray:
    """dS = P * (dP - D) (softmax backward, row-wise)."""
    return P * (dP - Di[:, None])


def _default_scale(D: int, scale) -> float:
    return 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)


def _row_slices(rows: np.ndarray, row_block: int):
    for s0 in range(0, rows.shape[0], row_block):
        yield rows[s0:s0 + row_block]


def _visible_range(vis: np.ndarray):
    cols = np.flatnonzero(vis.any(axis=0))
    if cols.size == 0:
        return None
    return int(cols[0]), int(cols[-1]) + 1


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Masked softmax pieces for a slice: (p unnormalised, m, l)."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    p = np.exp(s - np.where(has, m, 0.0)[:, None])
    l = p.sum(axis=1)
    return p, m, l


def _sink_logits(sink, Hq: int):
    """None (plain softmax) or the per-q-head sink logits z as an fp64 array [Hq]."""
    if sink is None:
        return None
    z = as_f64(sink).reshape(-1)
    if z.shape[0] == 1:
        z = np.full(Hq, z[0])
    assert z.shape[0] == Hq
    return z


def _sink_weight(z, m, l):
    """exp(z - m) for the rows' key statistics (m, l); 0 without a sink, and 0 for rows
    that see no key (their output is 0 whatever the sink)."""
    if z is None:
        return np.zeros_like(l)
    return np.where(np.isfinite(m), np.exp(z - np.where(np.isfinite(m), m, 0.0)), 0.0)


def _bias_rows(bias, b, h, rows, c0, c1):
    """bias[b, h, rows, c0:c1] of a broadcastable [B|1, H|1, Sq|1, Skv|1] array, or 0."""
    if bias is None:
        return 0.0
    bb = bias[min(b, bias.shape[0] - 1), min(h, bias.shape[1] - 1)]
    r = bb[rows] if bb.shape[0] > 1 else bb[np.zeros_like(rows)]
    return r[:, c0:c1] if r.shape[1] > 1 else r


def _drop_rows(drop, b, h, rows, Skv):
    """Dropped pairs drop[b, h, rows, :] of a broadcastable boolean array, or none."""
    if drop is None:
        return np.zeros((len(rows), Skv), dtype=bool)
    dd = drop[min(b, drop.shape[0] - 1), min(h, drop.shape[1] - 1)]
    r = dd[rows] if dd.shape[0] > 1 else dd[np.zeros_like(rows)]
    return np.broadcast_to(r, (len(rows), Skv))


def forward(q, k, v, *, causal: bool, window=(-1, -1), scale=None, q_pos0: int = 0,
            kv_pos0: int = 0, rows=None, heads=None, row_block: int = 256, sink=None, bias=None,
            dropout=None):
    """Attention forward from the definition.

    q: [B, Sq, Hq, D]; k: [B, Skv, Hkv, D]; v: [B, Skv, Hkv, Dv] (torch or numpy, any
    float dtype).  Returns (o [B, Sq, Hq, Dv], m [B, Hq, Sq], l [B, Hq, Sq]) in fp64, with m in the
    natural-log units of the scaled logits.  ``rows`` / ``heads`` restrict the
    evaluation to sampled query rows / q heads; entries not evaluated are NaN.  ``sink``:
    None, or the sink logits z [Hq] (zeros for "off_by_one"); m and l exclude the sink.
    ``bias``: None, or an additive logit bias broadcastable to [B, Hq, Sq, Skv].
    ``dropout``: None, or a boolean array broadcastable to [B, Hq, Sq, Skv], True = dropped.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sc = _default_scale(D, scale)
    wl, wr = window
    z = _sink_logits(sink, Hq)
    bias = None if bias is None else as_f64(bias)
    drop = None if dropout is None else np.asarray(dropout, dtype=bool)
    fill = np.nan if (rows is not None or heads is not None) else 0.0
    o = np.full((B, Sq, Hq, v.shape[3]), fill)
    m = np.full((B, Hq, Sq), np.nan if fill != 0.0 else -np.inf)
    l = np.full((B, Hq, Sq), fill)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    kpos = kv_pos0 + np.arange(Skv)
    for b in range(B):
        for hq in heads:
            g = kv_head_of(hq, G)
            K, V = k[b, :, g, :], v[b, :, g, :]
            for r in _row_slices(rows, row_block):
                vis = visible(q_pos0 + r, kpos, causal, wl, wr)
                if bias is not None:
                    vis = vis & (_bias_rows(bias, b, hq, r, 0, Skv) > -np.inf)
                vis = vis & ~_drop_rows(drop, b, hq, r, Skv)
                rng = _visible_range(vis)
                if rng is None:
                    o[b, r, hq] = 0.0
                    m[b, hq, r] = -np.inf
                    l[b, hq, r] = 0.0
                    continue
                c0, c1 = rng
                s = scores(q[b, r, hq, :], K[c0:c1], sc) + _bias_rows(bias, b, hq, r, c0, c1)
                p, mr, lr = _softmax_rows(s, vis[:, c0:c1])
                denom = lr + _sink_weight(None if z is None else z[hq], mr, lr)
                denom = np.where(denom > 0, denom, 1.0)
                o[b, r, hq] = (p @ V[c0:c1]) / denom[:, None]
                m[b, hq, r] = mr
                l[b, hq, r] = lr
    return o, m, l


def probs(q, k, *, causal: bool, window=(-1, -1), scale=None, q_pos0: int = 0, kv_pos0: int = 0):
    """Full probability matrix P [B, Hq, Sq, Skv] (small shapes only)."""
    q, k = as_f64(q), as_f64(k)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    G = Hq // Hkv
    sc = _default_scale(D, scale)
    vis = visible(q_pos0 + np.arange(Sq), kv_pos0 + np.arange(Skv), causal, *window)
    P = np.zeros((B, Hq, Sq, Skv))
    for b in range(B):
        for hq in range(Hq):
            p, _, lr = _softmax_rows(scores(q[b, :, hq], k[b, :, kv_head_of(hq, G)], sc), vis)
            P[b, hq] = p / np.where(lr > 0, lr, 1.0)[:, None]
    return P


def backward(q, k, v, do, *, causal: bool, window=(-1, -1), scale=None, q_pos0: int = 0,
             kv_pos0: int = 0, row_block: int = 256, heads=None, batches=None, sink=None, bias=None,
             dropout=None):
    """Analytic gradient of ``forward`` contracted with dO.

    Returns (dq [B, Sq, Hq, D], dk [B, Skv, Hkv, D], dv [B, Skv, Hkv, Dv]) in fp64.
    D_i uses this function's own fp64 output O.  ``heads`` / ``batches`` restrict the
    evaluation to some q heads / batch entries: dq of the others is NaN, and dk, dv
    only collect the contributions of the evaluated q heads (complete for a kv head
    when all q heads of its group are listed).  With ``sink`` (logits z [Hq]) the
    gradient of z is returned too: (dq, dk, dv, dz [Hq]).
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    G = Hq // Hkv
    sc = _default_scale(D, scale)
    wl, wr = window
    z = _sink_logits(sink, Hq)
    dz = np.zeros(Hq)
    bias = None if bias is None else as_f64(bias)
    drop = None if dropout is None else np.asarray(dropout, dtype=bool)
    partial = heads is not None or batches is not None
    dq = np.full_like(q, np.nan) if partial else np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Sq)
    kpos = kv_pos0 + np.arange(Skv)
    for b in (range(B) if batches is None else batches):
        for hq in (range(Hq) if heads is None else heads):
            g = kv_head_of(hq, G)
            dq[b, :, hq] = 0.0
            K, V = k[b, :, g, :], v[b, :, g, :]
            for r in _row_slices(rows, row_block):
                vis = visible(q_pos0 + r, kpos, causal, wl, wr)
                if bias is not None:
                    vis = vis & (_bias_rows(bias, b, hq, r, 0, Skv) > -np.inf)
                vis = vis & ~_drop_rows(drop, b, hq, r, Skv)
                rng = _visible_range(vis)
                if rng is None:
                    continue
                c0, c1 = rng
                s = scores(q[b, r, hq], K[c0:c1], sc) + _bias_rows(bias, b, hq, r, c0, c1)
                p, mr, lr = _softmax_rows(s, vis[:, c0:c1])
                w_sink = _sink_weight(None if z is None else z[hq], mr, lr)
                denom = lr + w_sink
                denom = np.where(denom > 0, denom, 1.0)
                P = p / denom[:, None]
                O = P @ V[c0:c1]
                dO = do[b, r, hq]
                Di = (dO * O).sum(axis=1)
                dz[hq] -= float(((w_sink / denom) * Di).sum())
                dP = dO @ V[c0:c1].T
                dS = grad_scores(P, dP, Di)
                dq[b, r, hq] = sc * (dS @ K[c0:c1])
                dk[b, c0:c1, g] += sc * (dS.T @ q[b, r, hq])
                dv[b, c0:c1, g] += P.T @ dO
    return (dq, dk, dv) if z is None else (dq, dk, dv, dz)


def visible_pairs(Sq: int, Skv: int, *, causal: bool, window=(-1, -1), q_pos0: int = 0,
                  kv_pos0: int = 0) -> int:
    """Number of visible (query, key) pairs per (batch, q head), counted row by row."""
    total = 0
    kp0, kp1 = kv_pos0, kv_pos0 + Skv - 1
    wl, wr = window
    for i in range(Sq):
        qp = q_pos0 + i
        hi = kp1
        if causal:
            hi = min(hi, qp)
        if wr >= 0:
            hi = min(hi, qp + wr)
        lo = kp0
        if wl >= 0:
            lo = max(lo, qp - wl)
        total += max(0, hi - lo + 1)
    return total
