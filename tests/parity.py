"""Tolerances for comparing GPU results with the fp64 oracle.

bf16 outputs / gradients: |gpu - ref| <= 2e-2 + 2^-8 |ref| element-wise (the second
term is one bf16 rounding of the stored value, needed where |ref| >= 8 since the bf16
half-ulp there exceeds 2e-2), plus a relative Frobenius error <= 1e-2 so that the
absolute bound cannot pass vacuously on small outputs.
fp32: |gpu - ref| <= 1e-4 + 2^-24 |ref| and relative Frobenius <= 1e-5.
The relative Frobenius bound holds over the whole comparison and, for BSHD tensors
[B, S, H, D], separately for every (batch, head, block of rows): a block is one virtual
ring block of ``blocks`` rows (the whole sequence when not given), so that a wrong
result on late rows, whose outputs are small, cannot hide behind the early rows.
Statistics: m within 1e-3 (bf16) / 1e-4 (fp32) absolute, l within 1e-3 / 1e-4 relative;
rows without any visible key must read m = -inf, l = 0 on both sides.
"""
import numpy as np
import torch


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def tol(dtype):
    bf16 = dtype in ("bf16", torch.bfloat16)
    return (2e-2, 2.0 ** -8, 1e-2) if bf16 else (1e-4, 2.0 ** -24, 1e-5)


def _rel_frob(g, r):
    denom = np.linalg.norm(r)
    return np.linalg.norm(g - r) / denom if denom > 0 else np.linalg.norm(g - r)


def check_close(name, gpu, ref, dtype, sel=None, blocks=None, rows=None):
    """Element bound and relative Frobenius bound (see the module docstring).  For 4-D
    [B, S, H, D] inputs the Frobenius bound is also checked per (batch, head, row block):
    ``blocks`` rows per block (None: one block), ``rows`` the sequence position of each
    entry along axis 1 when the rows are a sample (default 0 .. S-1)."""
    g, r = to_np(gpu), to_np(ref)
    if sel is not None:
        g, r = g[sel], r[sel]
    atol, rt, frob = tol(dtype)
    assert np.isfinite(g[~np.isnan(r)]).all(), f"{name}: non-finite GPU values"
    worst = 0.0
    if g.ndim == 4:
        pos = np.arange(g.shape[1]) if rows is None else np.asarray(rows)
        assert pos.shape == (g.shape[1],), f"{name}: rows must give one position per entry of axis 1"
        blk = np.zeros_like(pos) if blocks is None else pos // blocks
        for bi in range(g.shape[0]):
            for c in np.unique(blk):
                at = blk == c
                for h in range(g.shape[2]):
                    gg, rr = g[bi, at, h], r[bi, at, h]
                    keep = ~np.isnan(rr)
                    if not keep.any():
                        continue
                    rel_b = _rel_frob(gg[keep], rr[keep])
                    worst = max(worst, rel_b)
                    assert rel_b <= frob, (f"{name}: relative Frobenius error {rel_b:.3e} > {frob} in batch {bi}, "
                                           f"head {h}, row block {c}")
    keep = ~np.isnan(r)
    g, r = g[keep], r[keep]
    assert g.size > 0, f"{name}: nothing to compare"
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = np.abs(g - r)
    bound = atol + rt * np.abs(r)
    bad = err > bound
    rel = _rel_frob(g, r)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {g.size} outside tolerance; max abs err "
                           f"{err.max():.3e}, max |ref| {np.abs(r).max():.3e}, rel frob {rel:.3e}")
    assert rel <= frob, f"{name}: relative Frobenius error {rel:.3e} > {frob}"
    return float(err.max()), float(max(rel, worst))


def check_stats(m_gpu, l_gpu, m_ref, l_ref, dtype, sel=None):
    mg, lg, mr, lr = to_np(m_gpu), to_np(l_gpu), to_np(m_ref), to_np(l_ref)
    if sel is not None:
        mg, lg, mr, lr = mg[sel], lg[sel], mr[sel], lr[sel]
    keep = ~np.isnan(mr)
    mg, lg, mr, lr = mg[keep], lg[keep], mr[keep], lr[keep]
    bf16 = dtype in ("bf16", torch.bfloat16)
    m_tol, l_tol = (1e-3, 1e-3) if bf16 else (1e-4, 1e-4)
    empty = np.isneginf(mr)
    assert np.array_equal(np.isneginf(mg), empty), "rows without visible keys differ"
    assert np.all(lg[empty] == 0)
    full = ~empty
    if full.any():
        dm = np.abs(mg[full] - mr[full]).max()
        dl = (np.abs(lg[full] - lr[full]) / lr[full]).max()
        assert dm <= m_tol, f"m: max abs err {dm:.3e}"
        assert dl <= l_tol, f"l: max rel err {dl:.3e}"


def check_sum(name, gpu, ref, abs_terms, dtype):
    """A per-head sum over many rows (the sink-logit gradient): |gpu - ref| <= atol +
    c * sum_i |term_i|.  Each term carries the relative error of one bf16 rounding (the
    stored output enters D_i) plus fp32 exponentials, so the bound scales with the sum of
    the absolute terms; c = 2^-6 (bf16) or 1e-5 (fp32) leaves a factor of two or more."""
    g, r, a = to_np(gpu), to_np(ref), to_np(abs_terms)
    bf16 = dtype in ("bf16", torch.bfloat16)
    atol, c = (2e-2, 2.0 ** -6) if bf16 else (1e-4, 1e-5)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = np.abs(g - r)
    bound = atol + c * a
    assert np.all(err <= bound), f"{name}: max abs err {err.max():.3e} (bound {bound[err.argmax()]:.3e})"
    return float(err.max())
