"""GPU parity of the dense path (attn_fwd / attn_bwd through the C ABI) against the
fp64 oracle, on seeded inputs.

* small shapes that span several tiles and end in a ragged tail, for every mask kind
  (causal, sliding window, right window, none), GQA, position offsets, Sq != Skv,
  virtual ring blocks, bf16 head dims 32/64/128 and the fp32 path;
* every workload at its full size, in the launch configuration bench.py times, checked
  on sampled heads / rows the oracle can compute;
* the step API (carry in / no finalize), determinism and the degenerate cases;
* a value head dim of its own (the TransformerEngine page's DeepSeek-style MLA case,
  q/k 128 and v 64): small shapes through every mask kind and both workgroup shapes,
  the step API, and the page's full-size shape on one sampled GQA group.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import dense
from parity import check_close, check_stats, check_sum

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rnd(shape, seed, dtype):
    return workloads.random_tensor(shape, seed, dtype=dtype)


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


SMALL = [
    # id, dtype, B, Sq, Skv, Hq, Hkv, D, causal, window, q_pos0, kv_pos0, kv_block
    ("bf16_d128_causal_gqa2_ragged", "bf16", 2, 300, 300, 4, 2, 128, True, (-1, -1), 0, 0, 0),
    ("bf16_d64_full_ragged", "bf16", 1, 333, 333, 2, 1, 64, False, (-1, -1), 0, 0, 0),
    ("bf16_d128_swa37_gqa4", "bf16", 1, 515, 515, 8, 2, 128, True, (37, 0), 0, 0, 0),
    ("bf16_d32_window_offsets", "bf16", 1, 200, 260, 2, 2, 32, False, (5, 7), 60, 0, 0),
    ("bf16_d128_ring4", "bf16", 1, 1024, 1024, 2, 2, 128, True, (-1, -1), 0, 0, 256),
    ("bf16_d128_ring_swa", "bf16", 1, 768, 768, 4, 1, 128, True, (100, 0), 0, 0, 128),
    ("bf16_d128_right_window", "bf16", 1, 190, 190, 2, 1, 128, False, (-1, 20), 0, 0, 0),
    ("bf16_d64_ring_tiny_blocks", "bf16", 1, 256, 256, 2, 2, 64, True, (-1, -1), 0, 0, 32),
    ("bf16_d128_gqa8_ragged", "bf16", 2, 97, 97, 16, 2, 128, True, (-1, -1), 0, 0, 0),
    ("bf16_d64_gqa16_swa", "bf16", 1, 260, 260, 16, 1, 64, True, (50, 0), 0, 0, 0),
    ("bf16_d128_cross_len_offsets", "bf16", 1, 200, 520, 4, 4, 128, False, (-1, -1), 320, 0, 130),
    ("bf16_d32_gqa4_causal_offsets", "bf16", 1, 150, 300, 8, 2, 32, True, (-1, -1), 150, 0, 0),
    ("f32_d32_causal_gqa2", "f32", 1, 256, 256, 4, 2, 32, True, (-1, -1), 0, 0, 64),
    # windowed (32-key tiles): ring blocks of 130 keys, so tiles start off a 32-key
    # boundary; a window 509 keys wide, the widest that still takes the windowed kernels
    ("bf16_d128_swa_unaligned_blocks", "bf16", 1, 650, 650, 4, 2, 128, True, (300, 0), 0, 0, 130),
    ("bf16_d64_window_509", "bf16", 1, 900, 900, 2, 2, 64, False, (400, 108), 0, 0, 0),
    ("f32_d64_swa_ragged", "f32", 2, 77, 77, 2, 1, 64, True, (9, 0), 0, 0, 0),
]


def small_inputs(case):
    _, dt, B, Sq, Skv, Hq, Hkv, D, *_ = case
    t = tdtype(dt)
    seed = zlib.crc32(case[0].encode()) % 10000
    return (rnd((B, Sq, Hq, D), seed, t), rnd((B, Skv, Hkv, D), seed + 1, t),
            rnd((B, Skv, Hkv, D), seed + 2, t), rnd((B, Sq, Hq, D), seed + 3, t))


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_forward(gpu, case):
    name, dt, B, Sq, Skv, Hq, Hkv, D, causal, window, qp0, kp0, kvb = case
    q, k, v, _ = small_inputs(case)
    o, m, l = gpu.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window,
                           q_pos0=qp0, kv_pos0=kp0, kv_block=kvb)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_backward(gpu, case):
    name, dt, B, Sq, Skv, Hq, Hkv, D, causal, window, qp0, kp0, kvb = case
    q, k, v, do = small_inputs(case)
    kw = dict(causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0)
    check_close("dq", dq, dq_r, dt)
    check_close("dk", dk, dk_r, dt)
    check_close("dv", dv, dv_r, dt)


MLA_SMALL = [
    # id, dtype, B, Sq, Skv, Hq, Hkv, D, Dv, causal, window, q_pos0, kv_pos0, kv_block
    ("mla_bf16_causal_gqa4_ragged", "bf16", 2, 300, 300, 8, 2, 128, 64, True, (-1, -1), 0, 0, 0),
    ("mla_bf16_swa37_gqa16", "bf16", 1, 515, 515, 16, 1, 128, 64, True, (37, 0), 0, 0, 0),
    ("mla_bf16_ring_offsets", "bf16", 1, 512, 768, 4, 4, 128, 64, True, (-1, -1), 256, 0, 128),
    ("mla_bf16_right_window", "bf16", 1, 190, 190, 2, 1, 128, 64, False, (-1, 20), 0, 0, 0),
    ("mla_bf16_swa_ring_blocks", "bf16", 1, 576, 576, 4, 1, 128, 64, True, (77, 0), 0, 0, 96),
    ("mla_f32_d64_v32", "f32", 1, 200, 200, 4, 2, 64, 32, True, (-1, -1), 0, 0, 0),
]


def mla_inputs(case):
    _, dt, B, Sq, Skv, Hq, Hkv, D, Dv, *_ = case
    t = tdtype(dt)
    seed = zlib.crc32(case[0].encode()) % 10000
    return (rnd((B, Sq, Hq, D), seed, t), rnd((B, Skv, Hkv, D), seed + 1, t),
            rnd((B, Skv, Hkv, Dv), seed + 2, t), rnd((B, Sq, Hq, Dv), seed + 3, t))


@pytest.mark.parametrize("case", MLA_SMALL, ids=[c[0] for c in MLA_SMALL])
def test_mla_head_dims(gpu, case):
    name, dt, B, Sq, Skv, Hq, Hkv, D, Dv, causal, window, qp0, kp0, kvb = case
    q, k, v, do = mla_inputs(case)
    kw = dict(causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    torch.cuda.synchronize()
    assert o.shape == (B, Sq, Hq, Dv) and dv.shape == (B, Skv, Hkv, Dv) and dk.shape == (B, Skv, Hkv, D)
    okw = dict(causal=causal, window=window, q_pos0=qp0, kv_pos0=kp0)
    o_r, m_r, l_r = dense.forward(q, k, v, **okw)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, **okw)
    check_close("dq", dq, dq_r, dt)
    check_close("dk", dk, dk_r, dt)
    check_close("dv", dv, dv_r, dt)


SINK_CASES = [
    # id, dtype, B, S, Hq, Hkv, D, Dv, causal, window, kv_block, softmax_type
    ("sink_learnable_bf16_causal_gqa4", "bf16", 2, 300, 8, 2, 128, 128, True, (-1, -1), 0, "learnable"),
    ("sink_off_by_one_bf16_swa37_gqa16", "bf16", 1, 515, 16, 1, 128, 128, True, (37, 0), 0, "off_by_one"),
    ("sink_learnable_bf16_mla_ring", "bf16", 1, 512, 4, 4, 128, 64, True, (-1, -1), 128, "learnable"),
    ("sink_learnable_bf16_d64_window", "bf16", 1, 333, 4, 1, 64, 64, False, (20, 5), 0, "learnable"),
    ("sink_learnable_f32_d64", "f32", 1, 200, 4, 2, 64, 64, True, (-1, -1), 0, "learnable"),
]


@pytest.mark.parametrize("case", SINK_CASES, ids=[c[0] for c in SINK_CASES])
def test_sink_softmax(gpu, case):
    """softmax_type off_by_one / learnable: output, statistics (of the keys alone),
    gradients and the sink-logit gradient against the oracle."""
    name, dt, B, S, Hq, Hkv, D, Dv, causal, window, kvb, stype = case
    t = tdtype(dt)
    seed = zlib.crc32(name.encode()) % 10000
    q, k, v, do = (rnd((B, S, Hq, D), seed, t), rnd((B, S, Hkv, D), seed + 1, t),
                   rnd((B, S, Hkv, Dv), seed + 2, t), rnd((B, S, Hq, Dv), seed + 3, t))
    z = 1.5 * rnd((Hq,), seed + 4, torch.float32) if stype == "learnable" else torch.zeros(Hq)
    sk = dict(softmax_type=stype, sink=z.to(DEV) if stype == "learnable" else None)
    kw = dict(causal=causal, window=window, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw, **sk)
    grads = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw, **sk)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=causal, window=window, sink=z)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    dq_r, dk_r, dv_r, dz_r = dense.backward(q, k, v, do, causal=causal, window=window, sink=z)
    for nm, g_, r_ in (("dq", grads[0], dq_r), ("dk", grads[1], dk_r), ("dv", grads[2], dv_r)):
        check_close(nm, g_, r_, dt)
    if stype == "learnable":
        # sum over rows of |P_sink,i D_i|, from the oracle's own output and statistics
        zn = z.double().numpy()[None, :, None]
        w = np.exp(zn - np.where(np.isfinite(m_r), m_r, 0.0)) * np.isfinite(m_r)
        p_sink = w / np.where(l_r + w > 0, l_r + w, 1.0)
        d_row = np.einsum("bshd,bshd->bhs", do.double().numpy(), o_r)
        check_sum("dsink", grads[3], dz_r, np.abs(p_sink * d_row).sum(axis=(0, 2)), dt)


BIAS_CASES = [
    # id, dtype, B, S, Hq, Hkv, D, Dv, causal, window, kv_block, bias shape, kind
    ("bias_full_bf16_causal_gqa2", "bf16", 2, 300, 4, 2, 128, 128, True, (-1, -1), 0, "bhij", "randn"),
    ("bias_keypad_bf16_full", "bf16", 2, 260, 4, 4, 64, 64, False, (-1, -1), 0, "b11j", "keypad"),
    ("bias_row_bf16_swa_gqa16", "bf16", 1, 515, 16, 1, 128, 128, True, (37, 0), 0, "1hi1", "randn"),
    ("bias_dead_rows_bf16_ring", "bf16", 1, 512, 4, 2, 128, 128, True, (-1, -1), 128, "b1ij", "deadrows"),
    ("bias_full_bf16_mla", "bf16", 1, 333, 4, 1, 128, 64, True, (-1, -1), 0, "bhij", "randn"),
    ("bias_full_f32_d64", "f32", 1, 200, 4, 2, 64, 64, True, (-1, -1), 0, "bhij", "randn"),
    ("bias_full_bf16_swa_vec4", "bf16", 1, 300, 4, 2, 128, 128, True, (64, 0), 0, "bhij", "randn"),
]


def make_bias(kind, shape_code, B, Hq, S, seed):
    dims = {"b": B, "h": Hq, "i": S, "j": S, "1": 1}
    shape = tuple(dims[c] for c in shape_code)
    if kind == "randn":
        return 2.0 * workloads.random_tensor(shape, seed, dtype=torch.float32)
    bias = torch.zeros(shape, dtype=torch.float32)
    if kind == "keypad":                       # the last 37 keys of every sequence are padding
        bias[..., S - 37:] = float("-inf")
    else:                                      # random -inf pairs and a few rows with no key at all
        g = torch.Generator().manual_seed(seed)
        bias[torch.rand(shape, generator=g) < 0.2] = float("-inf")
        bias[..., 5, :] = float("-inf")
        bias[..., 200:203, :] = float("-inf")
    return bias


@pytest.mark.parametrize("case", BIAS_CASES, ids=[c[0] for c in BIAS_CASES])
def test_additive_bias(gpu, case):
    """bpt.py's additive logit bias (broadcast shapes, -inf padding, rows with no key left)
    through the forward and backward kernels (both workgroup shapes, MLA dims, fp32)."""
    name, dt, B, S, Hq, Hkv, D, Dv, causal, window, kvb, shape_code, kind = case
    t = tdtype(dt)
    seed = zlib.crc32(name.encode()) % 10000
    q, k, v, do = (rnd((B, S, Hq, D), seed, t), rnd((B, S, Hkv, D), seed + 1, t),
                   rnd((B, S, Hkv, Dv), seed + 2, t), rnd((B, S, Hq, Dv), seed + 3, t))
    bias = make_bias(kind, shape_code, B, Hq, S, seed + 4)
    kw = dict(causal=causal, window=window, kv_block=kvb)
    qd, kd, vd, dod, bd = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), bias.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, bias=bd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, bias=bd, **kw)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=causal, window=window, bias=bias)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, causal=causal, window=window, bias=bias)
    check_close("dq", dq, dq_r, dt)
    check_close("dk", dk, dk_r, dt)
    check_close("dv", dv, dv_r, dt)


SHARED_BIAS = [
    # id, B, S, Hq, Hkv, D, causal, window: one N(0,1) offset per key shared by every row
    ("g16_causal_d64_s96", 1, 96, 16, 1, 64, True, (-1, -1)),
    ("g8_causal_d128_s300", 2, 300, 16, 2, 128, True, (-1, -1)),
    ("g16_window120_d128_s400", 1, 400, 16, 1, 128, True, (120, 0)),
    ("g8_full_d64_s200", 1, 200, 8, 1, 64, False, (-1, -1)),
]


def shared_bias_inputs(case):
    name, B, S, Hq, Hkv, D, causal, window = case
    seed = zlib.crc32(name.encode()) % 10000
    t = torch.bfloat16
    q, k, v, do = (rnd((B, S, Hq, D), seed, t), rnd((B, S, Hkv, D), seed + 1, t),
                   rnd((B, S, Hkv, D), seed + 2, t), rnd((B, S, Hq, D), seed + 3, t))
    return q, k, v, do, workloads.random_tensor((B, 1, 1, S), seed + 4)


@pytest.mark.parametrize("scale", [1.0])
@pytest.mark.parametrize("case", SHARED_BIAS, ids=[c[0] for c in SHARED_BIAS])
def test_key_shared_bias_gradients(gpu, case, scale):
    """A bias of one N(0, scale^2) value per key, shared by every row and head ("bpt.py"'s
    bias broadcast over heads and query rows): a few keys take a large share of the
    attention of every (row, head) pair of a GQA group, so their dv and dk sum hundreds of
    large P and dS terms.  With P and dS as bf16 pairs in dV and dK and D from o + o_lo
    the gradients stay within the bf16 bound; an fp64 model of P and dS rounded to bf16
    puts dv past it on the first three shapes.  (At scale 2 the third shape's dk leaves
    the bound on 3 of 51200 elements, by 2 %, where that model of the kernel's roundings
    stays at 0.66 of it: an error source the model lacks, not yet found.)"""
    name, B, S, Hq, Hkv, D, causal, window = case
    q, k, v, do, bias = shared_bias_inputs(case)
    bias = scale * bias
    kw = dict(causal=causal, window=window)
    qd, kd, vd, dod, bd = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), bias.to(DEV)
    o_lo = torch.empty_like(dod)
    o, m, l = gpu.attn_fwd(qd, kd, vd, bias=bd, o_lo=o_lo, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, bias=bd, o_lo=o_lo, **kw)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, bias=bias, **kw)
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


DROP_CASES = [
    # id, dtype, B, Sq, Skv, Hq, Hkv, D, Dv, causal, window, q_pos0, kv_block, dropout shape, p, with bias
    ("drop_bf16_causal_gqa2", "bf16", 2, 300, 300, 4, 2, 128, 128, True, (-1, -1), 0, 0, "bhij", 0.2, False),
    ("drop_bf16_swa_gqa16_headshared", "bf16", 1, 515, 515, 16, 1, 128, 128, True, (37, 0), 0, 0, "b1ij", 0.3, False),
    ("drop_bf16_ring_unaligned_blocks", "bf16", 1, 520, 520, 4, 2, 128, 128, True, (-1, -1), 0, 130, "1hij", 0.1, False),
    ("drop_bf16_cross_offsets", "bf16", 1, 200, 520, 4, 4, 64, 64, False, (-1, -1), 320, 0, "bhij", 0.25, False),
    ("drop_bf16_mla", "bf16", 1, 333, 333, 4, 1, 128, 64, True, (-1, -1), 0, 0, "bhij", 0.2, False),
    ("drop_bf16_with_bias", "bf16", 2, 260, 260, 4, 4, 64, 64, True, (-1, -1), 0, 0, "bhij", 0.15, True),
    ("drop_f32_d64", "f32", 1, 200, 200, 4, 2, 64, 64, True, (-1, -1), 0, 0, "bhij", 0.2, False),
    ("drop_bf16_swa_unaligned_bias", "bf16", 1, 390, 390, 4, 2, 128, 128, True, (90, 0), 0, 130, "bhij", 0.2, True),
]


@pytest.mark.parametrize("case", DROP_CASES, ids=[c[0] for c in DROP_CASES])
def test_dropout(gpu, case):
    """bpt.py's dropout as a packed Bernoulli array (dropped pairs leave the softmax):
    forward and backward against the oracle, for broadcast shapes, key tiles that start
    off a 32-key boundary (ring blocks of 130), position offsets, MLA dims, together with
    a bias, and fp32."""
    name, dt, B, Sq, Skv, Hq, Hkv, D, Dv, causal, window, qp0, kvb, dshape, pdrop, with_bias = case
    t = tdtype(dt)
    seed = zlib.crc32(name.encode()) % 10000
    q, k, v, do = (rnd((B, Sq, Hq, D), seed, t), rnd((B, Skv, Hkv, D), seed + 1, t),
                   rnd((B, Skv, Hkv, Dv), seed + 2, t), rnd((B, Sq, Hq, Dv), seed + 3, t))
    dims = {"b": B, "h": Hq, "i": Sq, "j": Skv, "1": 1}
    g = torch.Generator().manual_seed(seed + 4)
    drop = torch.rand(tuple(dims[c] for c in dshape), generator=g) < pdrop
    bias = 2.0 * workloads.random_tensor((B, Hq, Sq, Skv), seed + 5) if with_bias else None
    kw = dict(causal=causal, window=window, q_pos0=qp0, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    words = workloads.pack_bits(drop).to(DEV)
    gk = dict(kw, dropout=words, bias=None if bias is None else bias.to(DEV))
    o, m, l = gpu.attn_fwd(qd, kd, vd, **gk)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **gk)
    torch.cuda.synchronize()
    ok = dict(causal=causal, window=window, q_pos0=qp0, dropout=drop.numpy(), bias=bias)
    o_r, m_r, l_r = dense.forward(q, k, v, **ok)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, **ok)
    check_close("dq", dq, dq_r, dt)
    check_close("dk", dk, dk_r, dt)
    check_close("dv", dv, dv_r, dt)


def test_sink_carry_is_applied_once(gpu):
    """Two ring steps with the carry handed over: the sink enters only when the output is
    finalised, so the result equals one call and the oracle."""
    B, S, Hq, Hkv, D = 1, 384, 4, 2, 128
    t = torch.bfloat16
    q, k, v = rnd((B, S, Hq, D), 51, t), rnd((B, 2 * S, Hkv, D), 52, t), rnd((B, 2 * S, Hkv, D), 53, t)
    z = rnd((Hq,), 54, torch.float32)
    qd, kd, vd, zd = q.to(DEV), k.to(DEV), v.to(DEV), z.to(DEV)
    acc, m, l = gpu.attn_fwd(qd, kd[:, S:].contiguous(), vd[:, S:].contiguous(), causal=True, q_pos0=S,
                             kv_pos0=S, finalize=False, softmax_type="learnable", sink=zd)
    o, m, l = gpu.attn_fwd(qd, kd[:, :S].contiguous(), vd[:, :S].contiguous(), causal=True, q_pos0=S,
                           kv_pos0=0, carry_in=True, m=m, l=l, acc=acc, softmax_type="learnable", sink=zd)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, q_pos0=S, kv_pos0=0, sink=z)
    check_close("o (two steps)", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")


def full_inputs(name, with_dout=True):
    w = workloads.WORKLOADS[name]
    q, k, v, do = workloads.generate(w, with_dout=with_dout)
    return w, q, k, v, do


def launch_kw(w):
    return dict(causal=w.causal, window=w.window, query_chunk=w.query_chunk, key_chunk=w.key_chunk,
                kv_block=w.kv_block)


def oracle_kw(w):
    return dict(causal=w.causal, window=w.window)


def test_tiny_fp32_workload(gpu):
    w, q, k, v, do = full_inputs("tiny_causal_gqa_fp32")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, scale=w.scale, **launch_kw(w))
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, scale=w.scale, **launch_kw(w))
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, scale=w.scale, **oracle_kw(w))
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, scale=w.scale, **oracle_kw(w))
    for nm, a, b in (("o", o, o_r), ("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        check_close(nm, a, b, "f32")
    check_stats(m, l, m_r, l_r, "f32")


def test_ring_sim_full_size(gpu):
    """B1 S8192 H16 D128 causal, 8 virtual blocks: all rows of 3 heads (fwd), 2 heads (bwd)."""
    w, q, k, v, do = full_inputs("ring_sim_causal_s8192")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **launch_kw(w))
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **launch_kw(w))
    torch.cuda.synchronize()
    heads = [0, 7, 15]
    o_r, m_r, l_r = dense.forward(q, k, v, heads=heads, **oracle_kw(w))
    blk = w.kv_block
    check_close("o", o[:, :, heads], o_r[:, :, heads], "bf16", blocks=blk)
    check_stats(m[:, heads], l[:, heads], m_r[:, heads], l_r[:, heads], "bf16")
    bh = [3, 12]
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, heads=bh, **oracle_kw(w))
    check_close("dq", dq[:, :, bh], dq_r[:, :, bh], "bf16", blocks=blk)
    check_close("dk", dk[:, :, bh], dk_r[:, :, bh], "bf16", blocks=blk)      # G = 1: kv head = q head
    check_close("dv", dv[:, :, bh], dv_r[:, :, bh], "bf16", blocks=blk)


def unpack_bits(words, n):
    """int32 words [..., W] -> boolean [..., n] (bit j % 32 of word j / 32)."""
    u = words.numpy().view(np.uint32)
    bits = (u[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(u.shape[:-1] + (-1,))[..., :n].astype(bool)


def test_ring_full_size_bias_dropout(gpu):
    """The ring workload with the inputs of bench --bias keypad --dropout 0.1 (last S/16 keys
    at -inf; Bernoulli(0.1) drops drawn on the GPU and packed): two heads checked forward,
    one backward, against the oracle given the same drops."""
    w, q, k, v, do = full_inputs("ring_sim_causal_s8192")
    B, S, H = w.batch, w.seqlen, w.num_q_heads
    bias = torch.zeros((B, 1, 1, S), dtype=torch.float32)
    bias[..., S - S // 16:] = float("-inf")
    g = torch.Generator(device=DEV).manual_seed(w.seed + 102)
    words = torch.empty((1, H, S, (S + 31) // 32), dtype=torch.int32, device=DEV)
    for h in range(H):
        words[0, h] = workloads.pack_bits(torch.rand((S, S), generator=g, device=DEV) < 0.1)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    kw = dict(launch_kw(w), bias=bias.to(DEV), dropout=words)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    torch.cuda.synchronize()
    for h in (2, 9):
        drop = unpack_bits(words[0, h].cpu(), S)[None, None]
        o_r, m_r, l_r = dense.forward(q, k, v, heads=[h], bias=bias, dropout=drop, **oracle_kw(w))
        check_close(f"o head {h}", o[:, :, [h]], o_r[:, :, [h]], "bf16")
        check_stats(m[:, [h]], l[:, [h]], m_r[:, [h]], l_r[:, [h]], "bf16")
        if h == 9:
            dq_r, dk_r, dv_r = dense.backward(q, k, v, do, heads=[h], bias=bias, dropout=drop, **oracle_kw(w))
            check_close("dq", dq[:, :, [h]], dq_r[:, :, [h]], "bf16")
            check_close("dk", dk[:, :, [h]], dk_r[:, :, [h]], "bf16")      # G = 1
            check_close("dv", dv[:, :, [h]], dv_r[:, :, [h]], "bf16")


def test_ring_full_size_shared_bias(gpu):
    """The ring workload with the input of bench --bias shared: one N(0,1) fp32 bias matrix
    [1, 1, S, S] added to the scaled logits of every head.  Two heads forward, one backward,
    per virtual block, against the oracle given the same bias."""
    w, q, k, v, do = full_inputs("ring_sim_causal_s8192")
    S = w.seqlen
    bias = workloads.random_tensor((1, 1, S, S), w.seed + 101)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    kw = dict(launch_kw(w), bias=bias.to(DEV))
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    torch.cuda.synchronize()
    blk = w.kv_block
    for h in (4, 11):
        o_r, m_r, l_r = dense.forward(q, k, v, heads=[h], bias=bias, **oracle_kw(w))
        check_close(f"o head {h}", o[:, :, [h]], o_r[:, :, [h]], "bf16", blocks=blk)
        check_stats(m[:, [h]], l[:, [h]], m_r[:, [h]], l_r[:, [h]], "bf16")
    h = 11
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, heads=[h], bias=bias, **oracle_kw(w))
    check_close("dq", dq[:, :, [h]], dq_r[:, :, [h]], "bf16", blocks=blk)
    check_close("dk", dk[:, :, [h]], dk_r[:, :, [h]], "bf16", blocks=blk)      # G = 1
    check_close("dv", dv[:, :, [h]], dv_r[:, :, [h]], "bf16", blocks=blk)


def test_gqa_swa_full_size(gpu):
    """B2 S4096 Hq128 Hkv8 D128, window (128, 0): one full GQA group checked fwd and bwd."""
    w, q, k, v, do = full_inputs("gqa16_swa128_s4096")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **launch_kw(w))
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **launch_kw(w))
    torch.cuda.synchronize()
    group = 5
    heads = list(range(16 * group, 16 * group + 16))
    b = 1
    qs, ks, vs, dos = q[b:b + 1], k[b:b + 1], v[b:b + 1], do[b:b + 1]
    o_r, m_r, l_r = dense.forward(qs, ks, vs, heads=heads, **oracle_kw(w))
    check_close("o", o[b:b + 1, :, heads], o_r[:, :, heads], "bf16")
    check_stats(m[b:b + 1, heads], l[b:b + 1, heads], m_r[:, heads], l_r[:, heads], "bf16")
    dq_r, dk_r, dv_r = dense.backward(qs, ks, vs, dos, heads=heads, **oracle_kw(w))
    check_close("dq", dq[b:b + 1, :, heads], dq_r[:, :, heads], "bf16")
    check_close("dk", dk[b:b + 1, :, group], dk_r[:, :, group], "bf16")
    check_close("dv", dv[b:b + 1, :, group], dv_r[:, :, group], "bf16")


def test_mla_full_size(gpu):
    """B2 S4096 Hq128 Hkv8, q/k 128, v 64, causal: one full GQA group checked fwd and bwd."""
    w, q, k, v, do = full_inputs("mla_qk128_v64_s4096")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **launch_kw(w))
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **launch_kw(w))
    torch.cuda.synchronize()
    group, b = 3, 0
    heads = list(range(16 * group, 16 * group + 16))
    qs, ks, vs, dos = q[b:b + 1], k[b:b + 1], v[b:b + 1], do[b:b + 1]
    o_r, m_r, l_r = dense.forward(qs, ks, vs, heads=heads[::5], **oracle_kw(w))
    check_close("o", o[b:b + 1, :, heads[::5]], o_r[:, :, heads[::5]], "bf16")
    check_stats(m[b:b + 1, heads[::5]], l[b:b + 1, heads[::5]], m_r[:, heads[::5]], l_r[:, heads[::5]], "bf16")
    dq_r, dk_r, dv_r = dense.backward(qs, ks, vs, dos, heads=heads, **oracle_kw(w))
    check_close("dq", dq[b:b + 1, :, heads], dq_r[:, :, heads], "bf16")
    check_close("dk", dk[b:b + 1, :, group], dk_r[:, :, group], "bf16")
    check_close("dv", dv[b:b + 1, :, group], dv_r[:, :, group], "bf16")


def test_long_context_sampled_rows(gpu):
    """B1 S131072 Hq32 Hkv8 D128 causal, 32 virtual blocks of 4096: 16 rows of every
    virtual block (its first and last row and 14 drawn at random, 512 in all) on all 32 q
    heads, with the relative Frobenius bound per (head, virtual block) -- the outputs of
    late rows are small (inputs x 0.5), so the element bound alone would be vacuous."""
    w, q, k, v, _ = full_inputs("long_causal_s131072", with_dout=False)
    o, m, l = gpu.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **launch_kw(w))
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    blk = w.kv_block
    rows = []
    for c in range(w.seqlen // blk):
        rows += [c * blk, c * blk + blk - 1] + list(c * blk + 1 + g.choice(blk - 2, 14, replace=False))
    rows = np.array(sorted(rows), dtype=np.int64)
    assert rows.size == 512
    o_r, m_r, l_r = dense.forward(q, k, v, rows=rows, row_block=16, **oracle_kw(w))
    ri = torch.from_numpy(rows)
    check_close("o", o[:, ri.to(o.device)].cpu(), o_r[:, rows], "bf16", blocks=blk, rows=rows)
    check_stats(m[:, :, ri.to(m.device)], l[:, :, ri.to(l.device)], m_r[:, :, rows], l_r[:, :, rows], "bf16")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_step_api_carry_equals_single_call(gpu, dt):
    """Two ring steps (the later kv block first, as the ring visits them) with the carry
    handed over through m, l, acc equal one call over both blocks."""
    t = tdtype(dt)
    B, S, Hq, Hkv, D = 1, 512, 4, 2, (128 if dt == "bf16" else 32)
    q, k, v = rnd((B, S, Hq, D), 11, t), rnd((B, 2 * S, Hkv, D), 12, t), rnd((B, 2 * S, Hkv, D), 13, t)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    # queries occupy positions S..2S-1 (ring member 1), keys 0..2S-1 in two blocks
    acc, m, l = gpu.attn_fwd(qd, kd[:, S:].contiguous(), vd[:, S:].contiguous(), causal=True,
                             q_pos0=S, kv_pos0=S, finalize=False)
    o, m, l = gpu.attn_fwd(qd, kd[:, :S].contiguous(), vd[:, :S].contiguous(), causal=True,
                           q_pos0=S, kv_pos0=0, carry_in=True, m=m, l=l, acc=acc)
    o1, m1, l1 = gpu.attn_fwd(qd, kd, vd, causal=True, q_pos0=S, kv_pos0=0)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, q_pos0=S, kv_pos0=0)
    check_close("o (two steps)", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    check_close("o (one call)", o1, o_r, dt)


RING_BWD = [
    # id, dtype, S per block, Hq, Hkv, D, Dv, softmax
    ("bf16_d128_gqa2", "bf16", 192, 4, 2, 128, 128, "vanilla"),
    ("bf16_mla_split_dkdv_sink", "bf16", 160, 8, 2, 128, 64, "learnable"),
    ("f32_d64", "f32", 96, 4, 2, 64, 64, "vanilla"),
]


@pytest.mark.parametrize("case", RING_BWD, ids=[c[0] for c in RING_BWD])
def test_ring_backward_steps_accumulate(gpu, case):
    """The backward ring on one GPU ("bpt.py", _ring_attention_bwd): two query blocks and
    two key blocks of a causal sequence, one attn_bwd call per (query block, key block) pair
    in ring order with ATTN_BWD_ACCUMULATE, adding into the query block's fp32 dq and the key
    block's fp32 dk, dv (the sink gradient once per query block).  Equal to the oracle and
    to the single call over the whole sequence."""
    name, dt, S, Hq, Hkv, D, Dv, softmax = case
    t = tdtype(dt)
    seed = zlib.crc32(name.encode()) % 10000
    B, N = 1, 2
    q, k, v, do = (rnd((B, N * S, Hq, D), seed, t), rnd((B, N * S, Hkv, D), seed + 1, t),
                   rnd((B, N * S, Hkv, Dv), seed + 2, t), rnd((B, N * S, Hq, Dv), seed + 3, t))
    z = rnd((Hq,), seed + 4, torch.float32) if softmax == "learnable" else None
    sk = dict(softmax_type=softmax, sink=z.to(DEV) if z is not None else None)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, causal=True, **sk)
    single = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, causal=True, **sk)
    blk = lambda x, i: x[:, i * S:(i + 1) * S].contiguous()
    f32 = torch.float32
    dq = [torch.zeros((B, S, Hq, D), dtype=f32, device=DEV) for _ in range(N)]
    dk = [torch.zeros((B, S, Hkv, D), dtype=f32, device=DEV) for _ in range(N)]
    dv = [torch.zeros((B, S, Hkv, Dv), dtype=f32, device=DEV) for _ in range(N)]
    dz = torch.zeros((Hq,), dtype=f32, device=DEV)
    for i in range(N):                                   # query block i = ring member i
        mi, li = m[:, :, i * S:(i + 1) * S].contiguous(), l[:, :, i * S:(i + 1) * S].contiguous()
        for idx in range(N):                             # ring step: key block (i - idx) mod N
            j = (i - idx) % N
            extra = dict(dsink=dz) if (z is not None and idx == 0) else {}
            gpu.attn_bwd(blk(qd, i), blk(kd, j), blk(vd, j), blk(o, i), blk(dod, i), mi, li, causal=True,
                         q_pos0=i * S, kv_pos0=j * S, accumulate=True, out=(dq[i], dk[j], dv[j]), **sk, **extra)
    torch.cuda.synchronize()
    dq_all, dk_all, dv_all = torch.cat(dq, 1), torch.cat(dk, 1), torch.cat(dv, 1)
    ref = dense.backward(q, k, v, do, causal=True, sink=z)
    check_close("dq (ring steps)", dq_all, ref[0], dt, blocks=S)
    check_close("dk (ring steps)", dk_all, ref[1], dt, blocks=S)
    check_close("dv (ring steps)", dv_all, ref[2], dt, blocks=S)
    for nm, a_, b_ in (("dq", dq_all, single[0]), ("dk", dk_all, single[1]), ("dv", dv_all, single[2])):
        check_close(f"{nm} (ring steps vs one call)", a_, b_.double().cpu(), dt)
    if z is not None:
        np.testing.assert_allclose(dz.cpu().numpy(), ref[3], atol=2e-2, rtol=2e-2)
        np.testing.assert_allclose(dz.cpu().numpy(), single[3].cpu().numpy(), atol=1e-4, rtol=1e-4)


def test_step_api_carry_with_bias(gpu):
    """Ring steps with a bias: each step gets the slice of the bias for its key block
    (a strided view), and the carried result equals one call with the whole bias, and
    the oracle (full [B, Hq, Sq, Skv] bias with -inf entries)."""
    B, S, Hq, Hkv, D = 1, 512, 4, 2, 128
    t = torch.bfloat16
    q, k, v = rnd((B, S, Hq, D), 21, t), rnd((B, 2 * S, Hkv, D), 22, t), rnd((B, 2 * S, Hkv, D), 23, t)
    bias = 2.0 * workloads.random_tensor((B, Hq, S, 2 * S), 24, dtype=torch.float32)
    bias[workloads.random_tensor((B, Hq, S, 2 * S), 25) > 1.5] = float("-inf")
    qd, kd, vd, bd = q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV)
    acc, m, l = gpu.attn_fwd(qd, kd[:, S:].contiguous(), vd[:, S:].contiguous(), causal=True,
                             q_pos0=S, kv_pos0=S, finalize=False, bias=bd[..., S:])
    o, m, l = gpu.attn_fwd(qd, kd[:, :S].contiguous(), vd[:, :S].contiguous(), causal=True,
                           q_pos0=S, kv_pos0=0, carry_in=True, m=m, l=l, acc=acc, bias=bd[..., :S])
    o1, m1, l1 = gpu.attn_fwd(qd, kd, vd, causal=True, q_pos0=S, kv_pos0=0, bias=bd)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, q_pos0=S, kv_pos0=0, bias=bias)
    check_close("o (two steps)", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")
    check_close("o (one call)", o1, o_r, "bf16")
    check_stats(m1, l1, m_r, l_r, "bf16")


def test_step_api_carry_with_dropout(gpu):
    """Ring steps with dropout: each step gets the words of its key block (a slice of the
    packed array at a word boundary), and the carried result equals one call and the
    oracle; the backward of the single call too."""
    B, S, Hq, Hkv, D = 1, 512, 4, 2, 128
    t = torch.bfloat16
    q, k, v = rnd((B, S, Hq, D), 41, t), rnd((B, 2 * S, Hkv, D), 42, t), rnd((B, 2 * S, Hkv, D), 43, t)
    do = rnd((B, S, Hq, D), 44, t)
    g = torch.Generator().manual_seed(45)
    drop = torch.rand((B, Hq, S, 2 * S), generator=g) < 0.2
    words = workloads.pack_bits(drop).to(DEV)                       # [B, Hq, S, 2S / 32]
    W = S // 32
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    acc, m, l = gpu.attn_fwd(qd, kd[:, S:].contiguous(), vd[:, S:].contiguous(), causal=True,
                             q_pos0=S, kv_pos0=S, finalize=False, dropout=words[..., W:])
    o, m, l = gpu.attn_fwd(qd, kd[:, :S].contiguous(), vd[:, :S].contiguous(), causal=True,
                           q_pos0=S, kv_pos0=0, carry_in=True, m=m, l=l, acc=acc, dropout=words[..., :W])
    o1, m1, l1 = gpu.attn_fwd(qd, kd, vd, causal=True, q_pos0=S, kv_pos0=0, dropout=words)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o1, dod, m1, l1, causal=True, q_pos0=S, kv_pos0=0, dropout=words)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, q_pos0=S, kv_pos0=0, dropout=drop.numpy())
    check_close("o (two steps)", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")
    check_close("o (one call)", o1, o_r, "bf16")
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, causal=True, q_pos0=S, kv_pos0=0, dropout=drop.numpy())
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


def test_bias_with_learnable_sink(gpu):
    """Bias and a learnable sink together: the sink joins the denominator of the biased
    logits; forward, gradients and the sink gradient against the oracle."""
    B, S, Hq, Hkv, D = 1, 300, 8, 2, 128
    t = torch.bfloat16
    q, k, v, do = (rnd((B, S, Hq, D), 31, t), rnd((B, S, Hkv, D), 32, t), rnd((B, S, Hkv, D), 33, t),
                   rnd((B, S, Hq, D), 34, t))
    z = 1.5 * rnd((Hq,), 35, torch.float32)
    bias = make_bias("keypad", "b11j", B, Hq, S, 36)
    kw = dict(causal=True, softmax_type="learnable", sink=z.to(DEV), bias=bias.to(DEV))
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv, dz = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, sink=z, bias=bias)
    check_close("o", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")
    dq_r, dk_r, dv_r, dz_r = dense.backward(q, k, v, do, causal=True, sink=z, bias=bias)
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")
    np.testing.assert_allclose(dz.cpu().numpy(), dz_r, atol=2e-2, rtol=2e-2)


def test_step_api_carry_mla(gpu):
    """The ring step API with a value head dim of its own: the carry acc has Dv columns."""
    B, S, Hq, Hkv, D, Dv = 1, 384, 4, 1, 128, 64
    t = torch.bfloat16
    q, k, v = rnd((B, S, Hq, D), 41, t), rnd((B, 2 * S, Hkv, D), 42, t), rnd((B, 2 * S, Hkv, Dv), 43, t)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    acc, m, l = gpu.attn_fwd(qd, kd[:, S:].contiguous(), vd[:, S:].contiguous(), causal=True,
                             q_pos0=S, kv_pos0=S, finalize=False)
    assert acc.shape == (B, S, Hq, Dv)
    o, m, l = gpu.attn_fwd(qd, kd[:, :S].contiguous(), vd[:, :S].contiguous(), causal=True,
                           q_pos0=S, kv_pos0=0, carry_in=True, m=m, l=l, acc=acc)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True, q_pos0=S, kv_pos0=0)
    check_close("o (two steps)", o, o_r, "bf16")
    check_stats(m, l, m_r, l_r, "bf16")


def test_no_finalize_carry_matches_oracle(gpu):
    B, S, H, D = 1, 256, 2, 64
    q, k, v = rnd((B, S, H, D), 21, torch.bfloat16), rnd((B, S, H, D), 22, torch.bfloat16), \
        rnd((B, S, H, D), 23, torch.bfloat16)
    acc, m, l = gpu.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, finalize=False)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, causal=True)
    check_stats(m, l, m_r, l_r, "bf16")
    # acc is the unnormalised numerator: acc / l must be the attention output
    check_close("acc/l", acc / l.transpose(1, 2)[..., None], o_r, "bf16")


@pytest.mark.parametrize("window,Dv", [((200, 0), 128), ((-1, -1), 128), ((-1, -1), 64)])
def test_backward_is_deterministic(gpu, window, Dv):
    """Bitwise repeatable: a windowed case (one dk/dv workgroup per key tile) and causal
    GQA cases whose q heads are shared out over several dk/dv workgroups (fp32 partials
    summed in a fixed order)."""
    B, S, Hq, Hkv, D = 1, 640, 8, 2, 128
    q, k, v, do = (rnd((B, S, Hq, D), 31, torch.bfloat16).to(DEV), rnd((B, S, Hkv, D), 32, torch.bfloat16).to(DEV),
                   rnd((B, S, Hkv, Dv), 33, torch.bfloat16).to(DEV), rnd((B, S, Hq, Dv), 34, torch.bfloat16).to(DEV))
    o, m, l = gpu.attn_fwd(q, k, v, causal=True, window=window)
    a = gpu.attn_bwd(q, k, v, o, do, m, l, causal=True, window=window)
    b = gpu.attn_bwd(q, k, v, o, do, m, l, causal=True, window=window)
    o2, _, _ = gpu.attn_fwd(q, k, v, causal=True, window=window)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(o, o2)


LOW_PART = [
    # id, B, S, Hq, Hkv, D, Dv, causal, window, kv_block, seed
    ("gqa8_window99_d64", 2, 211, 16, 2, 64, 64, True, (99, 0), 0, 4507),
    ("mla_gqa4_ring_ragged", 1, 300, 8, 2, 128, 64, True, (-1, -1), 100, 77),
    ("d128_full_window", 1, 257, 4, 4, 128, 128, False, (60, 20), 0, 91),
]


@pytest.mark.parametrize("case", LOW_PART, ids=[c[0] for c in LOW_PART])
def test_output_low_part(gpu, case):
    """o_lo, the output's low part ("bpt.py" keeps the output from before its cast to the
    input dtype for the backward): o is bitwise the same with and without it; o_lo is at
    most half a bf16 unit in the last place of o and zero where o is; o + o_lo is nearer
    the oracle's output than o; and the gradients that take it match the oracle.  The
    first shape's keys each collect about 800 (row, head) pairs (a GQA group of 8 under a
    causal window of 99 keys): there o alone puts enough of its rounding into D to leave
    the bf16 bound on one element of dk."""
    name, B, S, Hq, Hkv, D, Dv, causal, window, kvb, s = case
    t = torch.bfloat16
    q, k, v, do = rnd((B, S, Hq, D), s, t), rnd((B, S, Hkv, D), s + 1, t), rnd((B, S, Hkv, Dv), s + 2, t), \
        rnd((B, S, Hq, Dv), s + 3, t)
    kw = dict(causal=causal, window=window, kv_block=kvb)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o_lo = torch.full((B, S, Hq, Dv), float("nan"), dtype=t, device=DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, o_lo=o_lo, **kw)
    o_plain, _, _ = gpu.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, o_lo=o_lo, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "o must not depend on whether o_lo is written"
    hi, lo = o.cpu().double().numpy(), o_lo.cpu().double().numpy()
    assert np.isfinite(lo).all(), "o_lo must be written everywhere"
    nz = hi != 0
    assert (lo[~nz] == 0).all()
    half_ulp = np.exp2(np.floor(np.log2(np.abs(hi[nz]))) - 8)
    assert (np.abs(lo[nz]) <= half_ulp).all(), "o_lo exceeds half a bf16 ulp of o"
    o_r, _, _ = dense.forward(q, k, v, **kw_oracle(kw))
    rel = lambda x: np.linalg.norm(x - o_r) / np.linalg.norm(o_r)
    assert rel(hi + lo) < 0.8 * rel(hi), (rel(hi + lo), rel(hi))
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, **kw_oracle(kw))
    check_close("dq", dq, dq_r, "bf16")
    check_close("dk", dk, dk_r, "bf16")
    check_close("dv", dv, dv_r, "bf16")


def kw_oracle(kw):
    return dict(causal=kw["causal"], window=kw["window"])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rows_without_visible_keys(gpu, dt):
    t = tdtype(dt)
    B, Sq, Skv, H, D = 1, 200, 150, 2, 64
    q, k, v, do = rnd((B, Sq, H, D), 41, t), rnd((B, Skv, H, D), 42, t), rnd((B, Skv, H, D), 43, t), \
        rnd((B, Sq, H, D), 44, t)
    kw = dict(causal=True, q_pos0=0, kv_pos0=100)      # queries 0..99 precede every key
    o, m, l = gpu.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    dq, dk, dv = gpu.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o, do.to(DEV), m, l, **kw)
    torch.cuda.synchronize()
    o_r, m_r, l_r = dense.forward(q, k, v, **kw)
    check_close("o", o, o_r, dt)
    check_stats(m, l, m_r, l_r, dt)
    assert torch.all(o[:, :100] == 0) and torch.all(dq[:, :100] == 0)
    dq_r, dk_r, dv_r = dense.backward(q, k, v, do, **kw)
    check_close("dk", dk, dk_r, dt)
    check_close("dv", dv, dv_r, dt)


def test_empty_key_set_and_zero_sizes(gpu):
    q = rnd((1, 64, 2, 64), 51, torch.bfloat16).to(DEV)
    k = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device=DEV)
    o, m, l = gpu.attn_fwd(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(m)) and torch.all(l == 0)
    q0 = torch.empty((0, 64, 2, 64), dtype=torch.bfloat16, device=DEV)
    o0, _, _ = gpu.attn_fwd(q0, q0, q0)
    assert o0.shape == q0.shape
