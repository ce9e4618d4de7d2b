"""Exact top-n block selection over block means, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``select_block`` of the "AnnAttention" page ("Core code"), with the index
replaced by exact brute force:
  * the keys of one sequence are cut into blocks of ``block_size`` tokens; a block's
    key vector is the mean of its rows (the page inserts ``mean(bk)`` of each full
    block);
  * the page walks the query blocks in order, searches the index with every token
    of the block, and only then inserts the block's own mean (training mode), so a
    token in block i can select among blocks 0 .. i-1 only;
  * score(t, c) = q_t . mean_c (inner product); each token keeps its top
    min(top_n, i) blocks by (score descending, block index ascending on ties);
  * missing results are -1; the list is sorted ascending, so -1 entries come first.

Readings (the page shows neither the index construction nor the helpers): exact
inner product instead of HNSW's approximate search; a fresh index per sequence and
per call; ties go to the lower block index.  These readings are pinned only to
themselves -- parity unpinned against the original faiss-based code, which is not
reproducible from the page.

Decoding (the page's inference mode, ``training=False``, with the index kept across calls):
a block's mean enters the index only when the key cache has just reached the end of that
block, after the call's search, so a new token at position t still chooses among the
full blocks before its own block -- the same candidates as above.  ``q_pos0`` places the
query rows at positions q_pos0 .. q_pos0 + Sq - 1 of a key cache of any length Skv; the
means are those of the cache's full blocks (a mean is a function of its rows, so
recomputing them equals keeping them in an index).  The page's inference-mode loop is
garbled in the extracted text, so this reading is pinned only to itself (equality with
the full-sequence rows, brute force on the same reading): parity unpinned against the
page.

Precision: block means of bf16 inputs are exact in fp64 (a sum of 32 bf16 values fits
in 53 bits; dividing by 32 is exact), and fp64 dot products leave rounding of ~1e-16
relative, far below the score gaps of the workloads (``min_gap`` reports them).
"""
from __future__ import annotations

import numpy as np

from .dense import as_f64


def _flat(x):
    x = as_f64(x)
    if x.ndim == 4:                       # [B, S, H, D] -> joint embedding [B, S, H*D]
        x = x.reshape(x.shape[0], x.shape[1], -1)
    return x


def block_means(k, block_size: int) -> np.ndarray:
    """[B, S, E] -> [B, S // block_size, E]: mean of each full block of rows."""
    k = _flat(k)
    B, S, E = k.shape
    nb = S // block_size
    return k[:, :nb * block_size].reshape(B, nb, block_size, E).sum(axis=2) / block_size


def rank_candidates(sc: np.ndarray) -> np.ndarray:
    """Per row, candidate indices by score descending; equal scores keep index order."""
    return np.argsort(-sc, axis=1, kind="stable")


def block_select(q, k, *, block_size: int, top_n: int, return_gap: bool = False, q_pos0: int = 0):
    """Selected block indices int32 [B, Sq, top_n] (ascending, -1 first) for query rows at
    positions q_pos0 .. q_pos0 + Sq - 1 of the key sequence k [B, Skv, E].

    With ``return_gap`` also returns the smallest gap between the top_n-th and the
    (top_n+1)-th score over all tokens that had more than top_n candidates.
    """
    q, k = _flat(q), _flat(k)
    B, Sq, E = q.shape
    means = block_means(k, block_size)
    out = np.full((B, Sq, top_n), -1, dtype=np.int32)
    min_gap = np.inf
    if Sq == 0:
        return (out, min_gap) if return_gap else out
    first, last = q_pos0 // block_size, (q_pos0 + Sq - 1) // block_size
    for b in range(B):
        for i in range(first, last + 1):              # blocks of query positions
            p0, p1 = max(i * block_size, q_pos0), min((i + 1) * block_size, q_pos0 + Sq)
            r0, r1 = p0 - q_pos0, p1 - q_pos0         # their query rows
            n_cand = min(i, means.shape[1])
            if n_cand == 0:
                continue                              # nothing inserted yet: all -1
            sc = q[b, r0:r1] @ means[b, :n_cand].T    # [tokens, candidates]
            order = rank_candidates(sc)                  # ties: lower index first
            keep = min(top_n, n_cand)
            chosen = np.sort(order[:, :keep], axis=1)
            out[b, r0:r1, top_n - keep:] = chosen
            if return_gap and n_cand > top_n:
                srt = np.take_along_axis(sc, order, axis=1)
                min_gap = min(min_gap, float((srt[:, top_n - 1] - srt[:, top_n]).min()))
    if return_gap:
        return out, min_gap
    return out
