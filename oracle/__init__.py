"""Plain CPU oracle for blockwise exact attention (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call it.  It shares no code with the HIP library; the only module both
sides use is ``workloads`` (seeded inputs, no attention arithmetic).

Sources (web pages, cited by title and section):
  * "bpt.py" (llm_large_context repository): ring attention and blockwise attention
    in JAX -- ``_ring_attention_fwd/_bwd``, ``_blockwise_attention_fwd/_bwd``,
    ``_chunk_attention_bias`` and the ``__main__`` self-test's ``reference_attn``.
  * "JAX: Single-GPU Attention with TransformerEngine", section 1 (native JAX BSHD
    GQA + SWA baseline: ``_repeat_kv_for_gqa``, ``_make_causal_swa_mask``,
    ``FlaxNativeGQAAttention``) and "Other attention knobs" (score scaling).
  * "AnnAttention" (StudyExchange), section "Core code": ``select_block`` and
    ``faiss_block_attention``.

Modules:
  dense      -- softmax(scale * Q K^T + mask) V, its statistics and its analytic
                gradient, straight from the definition.
  blockwise  -- the pages' blockwise recurrence (numerator / denominator / max carried
                across KV chunks, ring order over virtual blocks, causal chunk skip);
                used to pin that the carry reaches the plain definition.
  select     -- exact top-n block selection over block means.
  sparse     -- attention over the gathered candidate list (window ++ selected blocks).

Every function is pinned by tests in ``tests/test_oracle_*.py`` to something other
than itself (an independent library routine, closed forms, invariants, finite
differences, brute force, a hand-worked example).  Where a reading of the pages is
only pinned to that reading, the function's docstring says "parity unpinned".
"""
from . import dense, blockwise, select, sparse  # noqa: F401
