"""Seeded synthetic workloads shared by the oracle checks, the GPU tests and bench.py.

This module holds shapes and random-number generation only: none of the attention
arithmetic lives here. Both sides of every parity check receive the very same host
tensors produced below.

Recipe (the same for every workload):
  * ``torch.Generator().manual_seed(seed)`` on the CPU;
  * ``torch.randn`` in fp32, in the order q, k, v, dout, each of its full shape;
  * an optional multiplier (0.5 for the long-context workload);
  * a round-to-nearest-even cast to the workload's element type (bf16 or fp32).

Shapes are BSHD: q is [B, S, Hq, D], k is [B, S, Hkv, D], v is [B, S, Hkv, Dv] and o,
dout are [B, S, Hq, Dv], where Dv = D except in the MLA workload (q/k 128, v 64).  The
block-sparse workload stores 8 heads of 64 as one joint embedding of 512 per token
(the AnnAttention page flattens heads into one vector before attending), so its
tensors are viewed as [B, S, 1, 512].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # "bf16" or "f32"
    seed: int
    causal: bool = True
    window: tuple = (-1, -1)        # (left, right); -1 = unbounded
    query_chunk: int = 0            # 0 -> whole sequence
    key_chunk: int = 0
    kv_block: int = 0               # virtual ring block; 0 -> one block
    input_scale: float = 1.0
    backward: bool = True
    # block-sparse only
    sparse: bool = False
    block_size: int = 0
    top_n: int = 0
    sparse_window: int = 0
    head_dim_v: int = 0             # 0 -> head_dim
    note: str = ""

    @property
    def dv(self) -> int:
        return self.head_dim_v or self.head_dim

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # fp32 tiny case: 4 q heads share 2 kv heads, chunks of 64.
    "tiny_causal_gqa_fp32": Workload(
        "tiny_causal_gqa_fp32", batch=1, seqlen=256, num_q_heads=4, num_kv_heads=2,
        head_dim=32, dtype="f32", seed=0, causal=True, query_chunk=64, key_chunk=64,
        note="B1 S256 Hq4 Hkv2 D32 fp32 causal, chunks 64"),
    # One GPU's ring: 8 virtual KV blocks of 1024 visited in ring order.
    "ring_sim_causal_s8192": Workload(
        "ring_sim_causal_s8192", batch=1, seqlen=8192, num_q_heads=16, num_kv_heads=16,
        head_dim=128, dtype="bf16", seed=1, causal=True, query_chunk=512, key_chunk=512,
        kv_block=1024, note="B1 S8192 H16 D128 bf16 causal, 8 virtual blocks of 1024"),
    # GQA group 16 with a causal sliding window of 128 to the left.
    "gqa16_swa128_s4096": Workload(
        "gqa16_swa128_s4096", batch=2, seqlen=4096, num_q_heads=128, num_kv_heads=8,
        head_dim=128, dtype="bf16", seed=2026, causal=True, window=(128, 0),
        note="B2 S4096 Hq128 Hkv8 D128 bf16 causal window (128,0)"),
    # Long context: 32 virtual blocks of 4096, forward only, inputs scaled by 0.5.
    "long_causal_s131072": Workload(
        "long_causal_s131072", batch=1, seqlen=131072, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", seed=3, causal=True, query_chunk=4096, key_chunk=4096,
        kv_block=4096, input_scale=0.5, backward=False,
        note="B1 S131072 Hq32 Hkv8 D128 bf16 causal, 32 virtual blocks of 4096, fwd"),
    # DeepSeek-style MLA head dims behind the projections: q/k 128, v 64, causal, GQA 16
    # (the TransformerEngine page, section 4, on its section-1 shape).
    "mla_qk128_v64_s4096": Workload(
        "mla_qk128_v64_s4096", batch=2, seqlen=4096, num_q_heads=128, num_kv_heads=8,
        head_dim=128, head_dim_v=64, dtype="bf16", seed=2027, causal=True,
        note="B2 S4096 Hq128 Hkv8 q/k 128 v 64 bf16 causal"),
    # Block-sparse: per-token exact top-8 over earlier 32-token block means + window 32.
    "block_sparse_top8_s8192": Workload(
        "block_sparse_top8_s8192", batch=4, seqlen=8192, num_q_heads=1, num_kv_heads=1,
        head_dim=512, dtype="bf16", seed=4, causal=True, backward=False, sparse=True,
        block_size=32, top_n=8, sparse_window=32,
        note="B4 S8192 8x64 heads as joint E=512, bf16, top-8 of 32-token blocks + window 32"),
}


def generate(w: Workload, *, with_dout: bool | None = None):
    """Return (q, k, v, dout) as CPU tensors of the workload's dtype (dout may be None)."""
    if with_dout is None:
        with_dout = w.backward
    g = torch.Generator().manual_seed(w.seed)
    B, S, Hq, Hkv, D, Dv = w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dv
    out = []
    for shape in ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, Dv)):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.input_scale != 1.0:
            t.mul_(w.input_scale)
        out.append(t.to(w.torch_dtype))
    dout = None
    if with_dout:
        t = torch.randn((B, S, Hq, Dv), generator=g, dtype=torch.float32)
        if w.input_scale != 1.0:
            t.mul_(w.input_scale)
        dout = t.to(w.torch_dtype)
    return out[0], out[1], out[2], dout


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same kind of mask, dtype and head grouping)."""
    return w.with_(**kw)


def pack_bits(mask: torch.Tensor) -> torch.Tensor:
    """Boolean [..., N] -> int32 words [..., ceil(N / 32)], bit j % 32 of word j / 32 = mask[..., j]
    (the packed dropout bits the library reads)."""
    N = mask.shape[-1]
    W = (N + 31) // 32
    m = torch.zeros(mask.shape[:-1] + (W * 32,), dtype=torch.int32, device=mask.device)
    m[..., :N] = mask.to(torch.int32)
    # disjoint bits: the int32 sum is their OR (bit 31 wraps to the sign bit)
    shifts = torch.arange(32, dtype=torch.int32, device=mask.device)
    return (m.reshape(mask.shape[:-1] + (W, 32)) << shifts).sum(-1, dtype=torch.int32)


def random_tensor(shape, seed: int, dtype=torch.float32, scale: float = 1.0):
    """Standalone seeded N(0, scale^2) tensor (used for edge-case shapes in tests)."""
    g = torch.Generator().manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)
