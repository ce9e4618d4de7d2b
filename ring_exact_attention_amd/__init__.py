"""Blockwise exact softmax attention for MI355X (gfx950): Python binding of libattn.so.

This module only marshals arguments: it checks tensor shapes/dtypes, allocates the
outputs with torch on the tensors' device, and calls the C ABI declared in
``include/attn.h`` on the current torch stream.  Every step of the computation runs
in the HIP kernels of ``libattn.so``; there is no fallback.  If the library has not
been built (``python -m ring_exact_attention_amd.build``), importing works but every
call raises.

Entry points (names as in the C ABI):
  attn_fwd(q, k, v, ...)                 -> (o, m, l)      or (acc, m, l) without finalize
  attn_bwd(q, k, v, o, dout, m, l, ...)  -> (dq, dk, dv)
  attn_bwd_noalloc(q, k, v, o, dout, m, l, out=(dq, dk, dv), ...)  (static scratch)
  block_select(q, k, block_size, top_n)  -> idx int32 [B, S, top_n]
  attn_fwd_sparse(q, k, v, idx, ...)     -> (o, m, l)      (attn_fwd with sel_idx)
  attn_bwd_sparse(q, k, v, idx, o, dout, m, l, ...) -> (dq, dk, dv)  (attn_bwd with sel_idx)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = 0, -1, -2, -3, -4
ATTN_BF16, ATTN_F32 = 0, 1
ATTN_CARRY_IN, ATTN_NO_FINALIZE = 1, 2
ATTN_BWD_SKIP_DQ, ATTN_BWD_SKIP_DKDV, ATTN_BWD_REUSE_STATS, ATTN_BWD_ACCUMULATE = 8, 16, 32, 64
ATTN_SOFTMAX_VANILLA, ATTN_SOFTMAX_OFF_BY_ONE, ATTN_SOFTMAX_LEARNABLE = 0, 1, 2
_SOFTMAX_TYPES = {"vanilla": ATTN_SOFTMAX_VANILLA, "off_by_one": ATTN_SOFTMAX_OFF_BY_ONE,
                  "learnable": ATTN_SOFTMAX_LEARNABLE}


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_kv", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("kv_pos0", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("query_chunk", ctypes.c_int32),
        ("key_chunk", ctypes.c_int32),
        ("kv_block", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("sel_idx", ctypes.c_void_p),
        ("top_n", ctypes.c_int32),
        ("sel_block", ctypes.c_int32),
        ("sparse_window", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("softmax_type", ctypes.c_int32),
        ("sink", ctypes.c_void_p),
        ("dsink", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("bias_stride", ctypes.c_int64 * 4),
        ("drop_mask", ctypes.c_void_p),
        ("drop_stride", ctypes.c_int64 * 3),
        ("o_lo", ctypes.c_void_p),
    ]


class SelectParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("embed", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_n", ctypes.c_int32),
        ("means_cached", ctypes.c_int32),
        ("seqlen_kv", ctypes.c_int32),
        ("q_pos0", ctypes.c_int32),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libattn status {status}: {message}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_SIGNATURES = {
    "attn_fwd": (ctypes.c_int, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _P, _P]),
    "attn_bwd": (ctypes.c_int, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, ctypes.c_size_t, _P]),
    "attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AttnParams)]),
    "attn_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AttnParams)]),
    "block_select": (ctypes.c_int, [ctypes.POINTER(SelectParams), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "block_select_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SelectParams)]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_abi_version": (ctypes.c_uint32, []),
}


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m ring_exact_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, lib().attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _softmax_code(softmax_type, sink):
    if softmax_type not in _SOFTMAX_TYPES:
        raise ValueError(f"softmax_type must be one of {sorted(_SOFTMAX_TYPES)}")
    code = _SOFTMAX_TYPES[softmax_type]
    if (code == ATTN_SOFTMAX_LEARNABLE) != (sink is not None):
        raise ValueError("sink (fp32 [num_q_heads]) is given exactly when softmax_type='learnable'")
    return code


def make_params(q, k, *, causal=True, window=(-1, -1), scale=None, query_chunk=0, key_chunk=0,
                kv_block=0, q_pos0=0, kv_pos0=0, flags=0, head_dim_v=0, softmax_type="vanilla",
                sink=None, bias=None, dropout=None, o_lo=None) -> AttnParams:
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head_dim")
    p = AttnParams()
    p.struct_size = ctypes.sizeof(AttnParams)
    p.dtype = _dtype_code(q)
    p.batch, p.seqlen_q, p.seqlen_kv = B, Sq, Skv
    p.num_q_heads, p.num_kv_heads, p.head_dim = Hq, Hkv, D
    p.head_dim_v = 0 if head_dim_v in (0, D) else int(head_dim_v)
    p.softmax_type = _softmax_code(softmax_type, sink)
    if sink is not None:
        _need(sink, "sink", torch.float32, q.device)
        if sink.shape != (Hq,):
            raise ValueError(f"sink must be [num_q_heads] = [{Hq}]")
        p.sink = sink.data_ptr()
    if bias is not None:
        # additive logit bias broadcastable to [B, Hq, Sq, Skv]: strides of the expanded view
        if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or bias.device != q.device:
            raise TypeError("bias must be a float32 tensor on q's device")
        if bias.dim() != 4:
            raise ValueError("bias must have 4 dims broadcastable to [B, Hq, Sq, Skv]")
        view = bias.expand(B, Hq, Sq, Skv)
        p.bias = bias.data_ptr()
        for d in range(4):
            p.bias_stride[d] = view.stride(d) if view.shape[d] > 1 else 0
    if dropout is not None:
        # packed dropout bits [B|1, Hq|1, Sq|1, W >= ceil(Skv / 32)] int32 words, bit j % 32 of
        # word j / 32 = pair (i, j) dropped (workloads.pack_bits builds them)
        if not isinstance(dropout, torch.Tensor) or dropout.dtype != torch.int32 or dropout.device != q.device:
            raise TypeError("dropout must be an int32 tensor of packed bits on q's device")
        W = (Skv + 31) // 32
        if dropout.dim() != 4 or dropout.shape[3] < W or dropout.stride(3) != 1:
            raise ValueError(f"dropout must be [B|1, Hq|1, Sq|1, >= {W}] words, contiguous in the last dim")
        view = dropout.expand(B, Hq, Sq, dropout.shape[3])
        p.drop_mask = dropout.data_ptr()
        for d in range(3):
            p.drop_stride[d] = view.stride(d) if view.shape[d] > 1 else 0
    if o_lo is not None:
        # the output's low part, bf16 [B, Sq, Hq, Dv] like o (attn_fwd writes it, attn_bwd reads it)
        Dv = head_dim_v if head_dim_v else D
        _need(o_lo, "o_lo", torch.bfloat16, q.device)
        if q.dtype != torch.bfloat16 or o_lo.shape != (B, Sq, Hq, Dv):
            raise ValueError(f"o_lo applies to bf16 attention and must be [B, Sq, Hq, Dv] = {(B, Sq, Hq, Dv)}")
        p.o_lo = o_lo.data_ptr()
    p.q_pos0, p.kv_pos0 = int(q_pos0), int(kv_pos0)
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.scale = 0.0 if scale is None else float(scale)
    p.query_chunk, p.key_chunk, p.kv_block = int(query_chunk), int(key_chunk), int(kv_block)
    p.flags = int(flags)
    return p


def attn_fwd(q, k, v, *, causal=True, window=(-1, -1), scale=None, query_chunk=0, key_chunk=0,
             kv_block=0, q_pos0=0, kv_pos0=0, m=None, l=None, acc=None, carry_in=False,
             finalize=True, out=None, softmax_type="vanilla", sink=None, bias=None, dropout=None,
             o_lo=None):
    """Forward attention.  q [B, Sq, Hq, D], k [B, Skv, Hkv, D], v [B, Skv, Hkv, Dv] on the GPU
    (Dv = D, or the MLA pair D 128 / Dv 64).

    Returns (o, m, l) with o [B, Sq, Hq, Dv]; with ``finalize=False`` returns (acc, m, l)
    where acc is the fp32 unnormalised numerator.  ``carry_in=True`` resumes from the
    given m, l, acc.  ``softmax_type`` "off_by_one" / "learnable" (with ``sink``, fp32
    [Hq] logits) adds exp(z_h) to each row's denominator when the output is finalised.
    ``bias``: fp32 additive logit bias broadcastable to [B, Hq, Sq, Skv] (-inf masks).
    ``dropout``: packed int32 dropout bits [B|1, Hq|1, Sq|1, ceil(Skv/32)] (see
    workloads.pack_bits); a set bit drops the pair from the softmax.  Pass the same
    tensor to attn_bwd.  ``o_lo``: a bf16 tensor shaped like o that a finalising call
    fills with the output's low part (fp32 output minus o, rounded); attn_bwd given it
    forms its row dot products D from the fp32 output instead of the rounded o.
    """
    _need(q, "q")
    _need(k, "k", q.dtype, q.device)
    _need(v, "v", q.dtype, q.device)
    if v.shape[:3] != k.shape[:3]:
        raise ValueError("k and v must agree on batch, length and heads")
    B, Sq, Hq, D = q.shape
    Dv = v.shape[3]
    flags = (ATTN_CARRY_IN if carry_in else 0) | (0 if finalize else ATTN_NO_FINALIZE)
    p = make_params(q, k, causal=causal, window=window, scale=scale, query_chunk=query_chunk,
                    key_chunk=key_chunk, kv_block=kv_block, q_pos0=q_pos0, kv_pos0=kv_pos0, flags=flags,
                    head_dim_v=Dv, softmax_type=softmax_type, sink=sink, bias=bias, dropout=dropout,
                    o_lo=o_lo if finalize else None)
    dev = q.device
    if m is None:
        m = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    _need(m, "m", torch.float32, dev)
    _need(l, "l", torch.float32, dev)
    if (carry_in or not finalize) and acc is None:
        acc = torch.empty((B, Sq, Hq, Dv), dtype=torch.float32, device=dev)
    if acc is not None:
        _need(acc, "acc", torch.float32, dev)
    if acc is not None and acc.shape != (B, Sq, Hq, Dv):
        raise ValueError(f"acc must be [B, Sq, Hq, Dv] = {(B, Sq, Hq, Dv)}")
    o = None
    if finalize:
        o = out if out is not None else torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=dev)
        _need(o, "o", q.dtype, dev)
        if o.shape != (B, Sq, Hq, Dv):
            raise ValueError(f"o must be [B, Sq, Hq, Dv] = {(B, Sq, Hq, Dv)}")
    _check(lib().attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l),
                          _ptr(acc), _stream(q)))
    return (o, m, l) if finalize else (acc, m, l)


def bwd_workspace_bytes(q, k, **kw) -> int:
    p = make_params(q, k, **kw)
    return int(lib().attn_bwd_workspace_bytes(ctypes.byref(p)))


def attn_bwd(q, k, v, o, dout, m, l, *, causal=True, window=(-1, -1), scale=None, query_chunk=0,
             key_chunk=0, kv_block=0, q_pos0=0, kv_pos0=0, workspace=None, out=None,
             skip_dq=False, skip_dkdv=False, reuse_stats=False, softmax_type="vanilla", sink=None,
             dsink=None, bias=None, dropout=None, accumulate=False, o_lo=None):
    """Gradients (dq, dk, dv) of attn_fwd's output for upstream gradient dout.

    ``skip_dq`` / ``skip_dkdv`` compute only part of them (the skipped outputs are left
    untouched); ``reuse_stats`` takes D and the log-sum-exp from ``workspace`` as left
    by an earlier call with the same inputs.  With ``softmax_type="learnable"`` the
    gradient of the sink logits is returned as a fourth tensor (fp32 [Hq]; written by
    calls that compute dq).  ``accumulate``: one ring step of the backward pass -- ``out``
    holds fp32 dq, dk, dv (and ``dsink`` fp32) that this call adds its gradients into
    (zeros are allocated when they are not given).  ``o_lo``: the output's low part that
    attn_fwd wrote, for D from the fp32 output.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, q.dtype, q.device)
    _need(m, "m", torch.float32, q.device)
    _need(l, "l", torch.float32, q.device)
    B, Sq, Hq, _ = q.shape
    Dv = v.shape[3]
    if v.shape[:3] != k.shape[:3] or o.shape != (B, Sq, Hq, Dv) or dout.shape != o.shape:
        raise ValueError("v must match k except in its head dim, and o, dout must be [B, Sq, Hq, Dv]")
    kw = dict(causal=causal, window=window, scale=scale, query_chunk=query_chunk, key_chunk=key_chunk,
              kv_block=kv_block, q_pos0=q_pos0, kv_pos0=kv_pos0, head_dim_v=Dv, softmax_type=softmax_type,
              sink=sink, bias=bias, dropout=dropout, o_lo=o_lo)
    flags = ((ATTN_BWD_SKIP_DQ if skip_dq else 0) | (ATTN_BWD_SKIP_DKDV if skip_dkdv else 0) |
             (ATTN_BWD_REUSE_STATS if reuse_stats else 0) | (ATTN_BWD_ACCUMULATE if accumulate else 0))
    p = make_params(q, k, flags=flags, **kw)
    need = int(lib().attn_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        if reuse_stats:
            raise ValueError("reuse_stats needs the workspace of the earlier call")
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    learnable = softmax_type == "learnable"
    if learnable:
        if dsink is None:
            dsink = torch.zeros((Hq,), dtype=torch.float32, device=q.device)
        _need(dsink, "dsink", torch.float32, q.device)
        p.dsink = dsink.data_ptr()
    if accumulate:
        f32 = torch.float32
        dq, dk, dv = out if out is not None else (torch.zeros_like(q, dtype=f32), torch.zeros_like(k, dtype=f32),
                                                  torch.zeros_like(v, dtype=f32))
        for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
            _need(t, n, f32, q.device)
            if t.shape != ref.shape:
                raise ValueError(f"{n} must have shape {tuple(ref.shape)}")
    else:
        dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    _check(lib().attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(m),
                          _ptr(l), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(q)))
    return (dq, dk, dv, dsink) if learnable else (dq, dk, dv)


NOALLOC_SCRATCH_BYTES = 64 << 20     # ATTN_NOALLOC_SCRATCH_BYTES of attn.h


def attn_bwd_noalloc(q, k, v, o, dout, m, l, *, out, causal=True, window=(-1, -1), scale=None,
                     query_chunk=0, key_chunk=0, kv_block=0, q_pos0=0, kv_pos0=0, skip_dq=False,
                     skip_dkdv=False, reuse_stats=False, softmax_type="vanilla", sink=None, dsink=None,
                     bias=None, dropout=None, o_lo=None):
    """attn_bwd without a workspace (the library's static scratch; see attn.h): the caller
    passes the outputs ``out = (dq, dk, dv)`` (and ``dsink`` for a learnable sink), so this
    call allocates nothing.  Returns ``out``."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, q.dtype, q.device)
    _need(m, "m", torch.float32, q.device)
    _need(l, "l", torch.float32, q.device)
    dq, dk, dv = out
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _need(t, n, q.dtype, q.device)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have shape {tuple(ref.shape)}")
    flags = ((ATTN_BWD_SKIP_DQ if skip_dq else 0) | (ATTN_BWD_SKIP_DKDV if skip_dkdv else 0) |
             (ATTN_BWD_REUSE_STATS if reuse_stats else 0))
    p = make_params(q, k, causal=causal, window=window, scale=scale, query_chunk=query_chunk,
                    key_chunk=key_chunk, kv_block=kv_block, q_pos0=q_pos0, kv_pos0=kv_pos0, flags=flags,
                    head_dim_v=v.shape[3], softmax_type=softmax_type, sink=sink, bias=bias, dropout=dropout,
                    o_lo=o_lo)
    if dsink is not None:
        _need(dsink, "dsink", torch.float32, q.device)
        p.dsink = dsink.data_ptr()
    _check(lib().attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(m),
                                  _ptr(l), _ptr(dq), _ptr(dk), _ptr(dv), _stream(q)))
    return out


def _joint(x):
    """[B, S, H, D] or [B, S, E] -> [B, S, E] view (heads flattened into one embedding)."""
    return x.reshape(x.shape[0], x.shape[1], -1) if x.dim() == 4 else x


def _select_params(B, S, E, block_size, top_n, seqlen_kv, q_pos0, means_cached=0):
    p = SelectParams()
    p.struct_size = ctypes.sizeof(SelectParams)
    p.dtype = ATTN_BF16
    p.batch, p.seqlen, p.embed = B, S, E
    p.seqlen_kv, p.q_pos0 = seqlen_kv, int(q_pos0)
    p.block_size, p.top_n = int(block_size), int(top_n)
    p.means_cached = int(means_cached)
    return p


def select_workspace_bytes(B, S, E, *, block_size=32, top_n=8, seqlen_kv=None, q_pos0=0) -> int:
    """Bytes of device workspace block_select needs for these sizes (keep one of this size
    to carry the block means across decoding calls)."""
    p = _select_params(B, S, E, block_size, top_n, S if seqlen_kv is None else seqlen_kv, q_pos0)
    return int(lib().block_select_workspace_bytes(ctypes.byref(p)))


def block_select(q, k, *, block_size=32, top_n=8, workspace=None, out=None, q_pos0=0, means_cached=0):
    """Exact top-n earlier-block selection by block-mean inner product -> int32 [B, Sq, top_n].

    Query row r sits at position q_pos0 + r of the key sequence k [B, Skv, E] (decoding:
    new tokens against the key cache).  ``means_cached``: the first that many blocks'
    means are already in ``workspace`` from an earlier call on the same key rows (the
    same workspace tensor, batch, embedding, block size and cache length)."""
    q, k = _joint(q), _joint(k)
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    B, S, E = q.shape
    if k.shape[0] != B or k.shape[2] != E:
        raise ValueError("q and k must agree on batch and embedding")
    p = _select_params(B, S, E, block_size, top_n, k.shape[1], q_pos0, means_cached)
    need = int(lib().block_select_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", device=q.device)
    idx = out if out is not None else torch.empty((B, S, top_n), dtype=torch.int32, device=q.device)
    _need(idx, "out", torch.int32, q.device)
    if idx.shape != (B, S, top_n):
        raise ValueError(f"out must be [B, Sq, top_n] = {(B, S, top_n)}")
    _check(lib().block_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(idx), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(q)))
    return idx


def attn_fwd_sparse(q, k, v, idx, *, window=32, block_size=32, scale=None, out=None, q_pos0=0,
                    workspace=None):
    """Attention of every token over its zero-padded window ++ selected blocks.  Query row r
    sits at position q_pos0 + r of the key / value sequence (decoding: new tokens against
    the cache, with idx from block_select(..., q_pos0=q_pos0)).  ``workspace``: a uint8
    device tensor of at least attn_fwd_workspace_bytes (allocated here when None and the
    call would use it), or False to run without the split over steps."""
    q, k, v = _joint(q), _joint(k), _joint(v)
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(v, "v", torch.bfloat16, q.device)
    _need(idx, "idx", torch.int32, q.device)
    B, S, E = q.shape
    top_n = idx.shape[-1]
    if idx.shape != (B, S, top_n):
        raise ValueError("idx must be [B, S, top_n]")
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != E:
        raise ValueError("k, v must be [B, Skv, E] with q's batch and embedding")
    p = AttnParams()
    p.struct_size = ctypes.sizeof(AttnParams)
    p.dtype = ATTN_BF16
    p.batch, p.seqlen_q, p.seqlen_kv = B, S, k.shape[1]
    p.q_pos0 = int(q_pos0)
    p.num_q_heads = p.num_kv_heads = 1
    p.head_dim = E
    p.scale = 0.0 if scale is None else float(scale)
    p.sel_idx = idx.data_ptr()
    p.top_n, p.sel_block, p.sparse_window = int(top_n), int(block_size), int(window)
    o = out if out is not None else torch.empty_like(q)
    m = torch.empty((B, S), dtype=torch.float32, device=q.device)
    l = torch.empty((B, S), dtype=torch.float32, device=q.device)
    need = int(lib().attn_fwd_workspace_bytes(ctypes.byref(p))) if workspace is not False else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if need and (workspace.numel() * workspace.element_size() < need or workspace.device != q.device):
        raise ValueError(f"workspace of {need} bytes on q's device needed")
    ws = _ptr(workspace) if need else None
    _check(lib().attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l), ws,
                          _stream(q)))
    return o, m, l


def fwd_sparse_workspace_bytes(B, S, *, top_n, window=32, block_size=32, seqlen_kv=None, q_pos0=0):
    """attn_fwd_workspace_bytes for a sparse forward of B x S query rows (embed 512)."""
    p = AttnParams()
    p.struct_size = ctypes.sizeof(AttnParams)
    p.dtype = ATTN_BF16
    p.batch, p.seqlen_q = int(B), int(S)
    p.seqlen_kv = int(seqlen_kv if seqlen_kv is not None else S)
    p.q_pos0 = int(q_pos0)
    p.num_q_heads = p.num_kv_heads = 1
    p.head_dim = 512
    p.sel_idx = 1
    p.top_n, p.sel_block, p.sparse_window = int(top_n), int(block_size), int(window)
    return int(lib().attn_fwd_workspace_bytes(ctypes.byref(p)))


def attn_bwd_sparse(q, k, v, idx, o, dout, m, l, *, window=32, block_size=32, scale=None,
                    workspace=None, out=None):
    """Gradients (dq, dk, dv) of attn_fwd_sparse's output o for upstream gradient dout."""
    q, k, v, o, dout = _joint(q), _joint(k), _joint(v), _joint(o), _joint(dout)
    for t, nme in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, nme, torch.bfloat16, q.device)
    _need(idx, "idx", torch.int32, q.device)
    _need(m, "m", torch.float32, q.device)
    _need(l, "l", torch.float32, q.device)
    B, S, E = q.shape
    top_n = idx.shape[-1]
    if idx.shape != (B, S, top_n) or m.shape != (B, S) or l.shape != (B, S):
        raise ValueError("idx must be [B, S, top_n] and m, l [B, S]")
    p = AttnParams()
    p.struct_size = ctypes.sizeof(AttnParams)
    p.dtype = ATTN_BF16
    p.batch, p.seqlen_q, p.seqlen_kv = B, S, S
    p.num_q_heads = p.num_kv_heads = 1
    p.head_dim = E
    p.scale = 0.0 if scale is None else float(scale)
    p.sel_idx = idx.data_ptr()
    p.top_n, p.sel_block, p.sparse_window = int(top_n), int(block_size), int(window)
    need = int(lib().attn_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    _check(lib().attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(m), _ptr(l),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def flops_fwd(visible_pairs_per_head: int, heads: int, batch: int, head_dim: int) -> float:
    """Algorithmic forward flops: 4*D per visible (query, key) pair per q head."""
    return 4.0 * head_dim * visible_pairs_per_head * heads * batch


def flops_bwd(visible_pairs_per_head: int, heads: int, batch: int, head_dim: int) -> float:
    """Algorithmic backward flops: 10*D per visible pair (recompute S, dP, dV, dQ, dK)."""
    return 10.0 * head_dim * visible_pairs_per_head * heads * batch


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
