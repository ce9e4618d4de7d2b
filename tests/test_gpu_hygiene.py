"""Memory-safety and order-independence checks through the C ABI.

* Guard bands: every output (and the backward / selection workspaces) is a view into the
  middle of a larger buffer poisoned with NaN (or a sentinel for integers).  After the
  call the output holds no poison -- every element was written -- and the bands before
  and after it are untouched, so nothing was written out of bounds.
* Reversed workgroup order: with ATTN_REVERSE_WORKGROUPS=1 every kernel takes its grid's
  tasks from the last one down.  No workgroup may depend on another's progress or on the
  order of their writes, so every result must be bitwise the same.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096            # elements (or bytes) on each side


def rnd(shape, seed, dtype=torch.bfloat16):
    return workloads.random_tensor(shape, seed, dtype=dtype).to(DEV)


class Guarded:
    """A view of `shape` in the middle of a poisoned buffer."""

    def __init__(self, shape, dtype, fill):
        self.n = math.prod(shape)
        self.fill = fill
        self.buf = torch.full((self.n + 2 * GUARD,), fill, dtype=dtype, device=DEV)
        self.view = self.buf[GUARD:GUARD + self.n].view(shape)

    def _is_fill(self, x):
        if x.dtype.is_floating_point and math.isnan(self.fill):
            return torch.isnan(x.float())
        return x == self.fill

    def check(self, name):
        assert self._is_fill(self.buf[:GUARD]).all(), f"{name}: written before its start"
        assert self._is_fill(self.buf[GUARD + self.n:]).all(), f"{name}: written past its end"
        assert not self._is_fill(self.view).any(), f"{name}: elements left unwritten"


def dense_case(gpu, B, S, Hq, Hkv, D, Dv, dtype, seed, **kw):
    q, k, v, do = (rnd((B, S, Hq, D), seed, dtype), rnd((B, S, Hkv, D), seed + 1, dtype),
                   rnd((B, S, Hkv, Dv), seed + 2, dtype), rnd((B, S, Hq, Dv), seed + 3, dtype))
    nan = float("nan")
    o, m, l = Guarded((B, S, Hq, Dv), dtype, nan), Guarded((B, Hq, S), torch.float32, nan), \
        Guarded((B, Hq, S), torch.float32, nan)
    gpu.attn_fwd(q, k, v, out=o.view, m=m.view, l=l.view, **kw)
    acc, m2, l2 = Guarded((B, S, Hq, Dv), torch.float32, nan), Guarded((B, Hq, S), torch.float32, nan), \
        Guarded((B, Hq, S), torch.float32, nan)
    gpu.attn_fwd(q, k, v, acc=acc.view, m=m2.view, l=l2.view, finalize=False, **kw)
    need = max(gpu.bwd_workspace_bytes(q, k, head_dim_v=Dv, **kw), 256)
    ws = Guarded((need,), torch.uint8, 255)
    dq, dk, dv = Guarded(q.shape, dtype, nan), Guarded(k.shape, dtype, nan), Guarded(v.shape, dtype, nan)
    gpu.attn_bwd(q, k, v, o.view, do, m.view, l.view, workspace=ws.view, out=(dq.view, dk.view, dv.view), **kw)
    torch.cuda.synchronize()
    outs = {"o": o, "m": m, "l": l, "acc": acc, "m (carry)": m2, "l (carry)": l2, "dq": dq, "dk": dk, "dv": dv}
    return outs, ws


DENSE = [
    # id, B, S, Hq, Hkv, D, Dv, dtype, kw
    ("bf16_causal_gqa4_ragged_split_dkdv", 2, 333, 8, 2, 128, 128, torch.bfloat16, dict(causal=True)),
    ("bf16_ring_g1", 1, 1024, 2, 2, 128, 128, torch.bfloat16, dict(causal=True, kv_block=256)),
    ("bf16_g8_8wave", 1, 300, 16, 2, 128, 128, torch.bfloat16, dict(causal=True)),
    ("bf16_swa_mla", 1, 515, 8, 1, 128, 64, torch.bfloat16, dict(causal=True, window=(37, 0))),
    ("bf16_d32_full", 1, 200, 2, 2, 32, 32, torch.bfloat16, dict(causal=False)),
    ("f32_d64_causal", 1, 150, 4, 2, 64, 64, torch.float32, dict(causal=True)),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_dense_guard_bands(gpu, case):
    _, B, S, Hq, Hkv, D, Dv, dtype, kw = case
    outs, ws = dense_case(gpu, B, S, Hq, Hkv, D, Dv, dtype, 7, **kw)
    for name, g in outs.items():
        g.check(name)
    assert (ws.buf[:GUARD] == 255).all() and (ws.buf[GUARD + ws.n:] == 255).all(), "workspace: written out of bounds"


def sparse_case(gpu, B, S, seed, W=32, n=8):
    E, bs = 512, 32
    q, k, v, do = rnd((B, S, E), seed), rnd((B, S, E), seed + 1), rnd((B, S, E), seed + 2), rnd((B, S, E), seed + 3)
    sel_ws = Guarded((max(gpu.lib().block_select_workspace_bytes(_select_params(gpu, B, S, E, bs, n)), 256),),
                     torch.uint8, 255)
    idx = Guarded((B, S, n), torch.int32, -12345)
    gpu.block_select(q, k, block_size=bs, top_n=n, out=idx.view, workspace=sel_ws.view)
    o = Guarded((B, S, E), torch.bfloat16, float("nan"))
    _, m, l = gpu.attn_fwd_sparse(q, k, v, idx.view, window=W, block_size=bs, out=o.view)
    grads = tuple(Guarded((B, S, E), torch.bfloat16, float("nan")) for _ in range(3))
    gpu.attn_bwd_sparse(q, k, v, idx.view, o.view, do, m, l, window=W, block_size=bs,
                        out=tuple(g.view for g in grads))
    # decoding: a few tokens against the cache, with the split-step workspace
    T = 3
    qn = q[:, S - T:].contiguous()
    idn = Guarded((B, T, n), torch.int32, -12345)
    gpu.block_select(qn, k, block_size=bs, top_n=n, out=idn.view, q_pos0=S - T)
    on = Guarded((B, T, E), torch.bfloat16, float("nan"))
    gpu.attn_fwd_sparse(qn, k, v, idn.view, window=W, block_size=bs, out=on.view, q_pos0=S - T)
    torch.cuda.synchronize()
    return {"idx": idx, "o": o, "dq": grads[0], "dk": grads[1], "dv": grads[2], "idx (decode)": idn,
            "o (decode)": on}, sel_ws


def _select_params(gpu, B, S, E, bs, n):
    import ctypes
    p = gpu.SelectParams()
    p.struct_size = ctypes.sizeof(gpu.SelectParams)
    p.dtype = gpu.ATTN_BF16
    p.batch, p.seqlen, p.embed, p.block_size, p.top_n = B, S, E, bs, n
    p.seqlen_kv, p.q_pos0 = S, 0
    return ctypes.byref(p)


def test_sparse_guard_bands(gpu):
    outs, ws = sparse_case(gpu, 2, 320, 11)
    for name, g in outs.items():
        g.check(name)
    assert (ws.buf[:GUARD] == 255).all() and (ws.buf[GUARD + ws.n:] == 255).all(), "select workspace"


def _values(outs):
    return {k: g.view.clone() for k, g in outs.items()}


def _bitwise(a, b, what):
    for name in a:
        x, y = a[name], b[name]
        same = torch.equal(x, y) if not x.dtype.is_floating_point else \
            torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                        y.view(torch.int16 if y.element_size() == 2 else torch.int32))
        assert same, f"{what} {name}: differs with the workgroup order reversed"


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_dense_reversed_workgroup_order(gpu, case):
    _, B, S, Hq, Hkv, D, Dv, dtype, kw = case
    fwd_order = _values(dense_case(gpu, B, S, Hq, Hkv, D, Dv, dtype, 7, **kw)[0])
    os.environ["ATTN_REVERSE_WORKGROUPS"] = "1"
    try:
        rev_order = _values(dense_case(gpu, B, S, Hq, Hkv, D, Dv, dtype, 7, **kw)[0])
    finally:
        os.environ.pop("ATTN_REVERSE_WORKGROUPS", None)
    _bitwise(fwd_order, rev_order, case[0])


def test_sparse_reversed_workgroup_order(gpu):
    fwd_order = _values(sparse_case(gpu, 2, 320, 11)[0])
    os.environ["ATTN_REVERSE_WORKGROUPS"] = "1"
    try:
        rev_order = _values(sparse_case(gpu, 2, 320, 11)[0])
    finally:
        os.environ.pop("ATTN_REVERSE_WORKGROUPS", None)
    _bitwise(fwd_order, rev_order, "sparse")
