"""Plain CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark import this module; the GPU library never
calls it and shares no code with it (numpy and the forward oracle only).

"FlashAttention Analysis" (ryotta.opik.net), in its closing section on
where the method sits, notes that paged KV caches (PagedAttention, vLLM)
run the fused kernels inside; the pages give no layout.  Reading taken (the layout of common serving engines): the
cache of one layer is ``[num_pages, page_size, Hkv, d]``; sequence b owns
the pages ``page_table[b, 0], page_table[b, 1], ...`` in that order, so its
key row r lives in page ``page_table[b, r // page_size]`` at slot
``r % page_size``, and its first ``seqlen_k[b]`` rows are its keys.  The
queries of sequence b then attend to those rows exactly as in the forward
oracle (bottom-right causal alignment at its own last key).
"""
from __future__ import annotations

import numpy as np

from .attention import reference_attention

__all__ = ["paged_rows", "paged_attention", "kvlen_attention"]


def paged_rows(cache, page_table_row, n: int):
    """The first ``n`` key (or value) rows of one sequence, gathered from
    its pages in order: an array [n, Hkv, d]."""
    num_pages, page_size = cache.shape[0], cache.shape[1]
    rows = np.empty((n,) + cache.shape[2:], dtype=cache.dtype)
    for r in range(n):
        page = int(page_table_row[r // page_size])
        if not 0 <= page < num_pages:
            raise ValueError("page index out of range")
        rows[r] = cache[page, r % page_size]
    return rows


def paged_attention(q, k_cache, v_cache, page_table, seqlen_k, *,
                    causal: bool, scale: float, window=None):
    """q [B, Hq, Nq, d]; caches [num_pages, page_size, Hkv, d]; page_table
    [B, max_pages]; seqlen_k [B].  Returns (O [B, Hq, Nq, d], lse
    [B, Hq, Nq]) with each sequence attending to its own gathered rows; a
    sequence with no keys gets O = 0, lse = -inf."""
    B, Hq, Nq, d = q.shape
    O = np.zeros(q.shape)
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        n = int(seqlen_k[b])
        if n == 0:
            continue
        k = paged_rows(k_cache, page_table[b], n).transpose(1, 0, 2)[None]
        v = paged_rows(v_cache, page_table[b], n).transpose(1, 0, 2)[None]
        Ob, lb = reference_attention(q[b:b + 1], k, v, causal=causal,
                                     scale=scale, window=window)
        O[b], lse[b] = Ob[0], lb[0]
    return O, lse


def kvlen_attention(q, k, v, seqlen_k, *, causal: bool, scale: float,
                    window=None):
    """Attention over a padded cache of unequal lengths.  q [B, Hq, Nq, d];
    k, v [B, Hkv, Nk_max, d]; seqlen_k [B].  Sequence b attends to its
    first ``seqlen_k[b]`` key rows only, with the causal and window
    alignment taken at its own last key, the same rule as for the paged
    cache (the rows past its length are padding and never read).  Returns
    (O [B, Hq, Nq, d], lse [B, Hq, Nq]); a sequence with no keys gets
    O = 0, lse = -inf."""
    B, Hq, Nq, d = q.shape
    O = np.zeros(q.shape)
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        length = int(seqlen_k[b])
        if not 0 <= length <= k.shape[2]:
            raise ValueError("sequence length out of range")
        if length == 0:
            continue
        Ob, lb = reference_attention(q[b:b + 1], k[b:b + 1, :, :length],
                                     v[b:b + 1, :, :length], causal=causal,
                                     scale=scale, window=window)
        O[b], lse[b] = Ob[0], lb[0]
    return O, lse
