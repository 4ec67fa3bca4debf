"""Plain float64 CPU oracle for the fused exact attention forward.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark import this module.  The GPU library never
calls it, and it shares no code with the GPU path: it imports numpy only.

Every function takes float64 arrays (bf16 inputs decoded exactly beforehand)
and works in float64 throughout:

    q : [B, Hq, Nq, d]        k, v : [B, Hkv, Nk, d]
    O : [B, Hq, Nq, d]        lse  : [B, Hq, Nq]

Sources (pages are named by title; sections as printed on them):

* "FlashAttention Analysis" (ryotta.opik.net), section 1 (the problem:
  standard attention computes S = Q K^T, then P = softmax(S), then O = P V,
  materialising S and P) and section 2 (the memory hierarchy: scaling and
  masking are steps of that same pass).
* same page, section 3 "Tiling + Online Softmax": a Q block stays fixed
  while K/V blocks stream; per row a running max m and running sum l; when a
  block raises the max, l and the partial O are rescaled by exp(m - m_new);
  O is divided by l once at the end.  The result is exact, only the order of
  work changes.
* same page, "Flash-Decoding": the KV axis is split into chunks whose
  partial results are combined by a log-sum-exp reduction.
* FlashAttention version / GPU / training-cost guide (tool.smithlab.co.kr),
  section on attention memory during training: one fp32 logsumexp value per
  query row is what is kept for the backward pass; checklist: causal masking
  is a flag, and grouped-query attention passes the KV-head count instead of
  replicating K/V heads (Qwen3-4B: 32 query heads over 8 KV heads).

Readings where the pages are silent (each is a documented choice):

* GQA head mapping: query head ``hq`` reads KV head ``hq // (Hq // Hkv)``
  (contiguous groups); ``Hq`` must be a multiple of ``Hkv``.
* Causal alignment when Nq != Nk: bottom-right, i.e. key ``j`` is visible to
  query ``i`` iff ``j <= i + (Nk - Nq)``; for Nq == Nk this is the usual lower
  triangle, and a single query (decode) sees every key.
* lse is the natural-log logsumexp of the scaled, masked scores.
* A query row with no visible key (only causal with Nq > Nk) has O = 0 and
  lse = -inf.
* Sliding window (the training-cost guide's FAQ names sliding windows among
  the mask features of the fused kernels; the pages give no formula):
  ``window = (left, right)`` keeps key ``j`` visible to query ``i`` only if
  ``c - left <= j <= c + right`` with ``c = i + (Nk - Nq)`` the query's own
  position on the key axis (the same bottom-right alignment as causal); a
  negative bound is no bound on that side.  ``(-1, 0)`` is the causal mask,
  ``(-1, -1)`` no mask; the window combines with ``causal`` by intersection.
  Rows whose window holds no key get O = 0 and lse = -inf.
* Block-sparse attention ("FlashAttention Analysis", results of
  FlashAttention-1: extended with a block-sparse pattern, only the non-zero
  blocks of a mask are computed, an approximation faster than the exact
  one; the pages give no block size or mask format): ``block_mask`` [B, Hq, nqb, nkb] (or
  broadcastable) with blocks of ``block_size = (bq, bk)`` query rows and
  keys; key j is visible to query i only if block (i // bq, j // bk) is
  non-zero, intersected with the causal flag and any window.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask", "block_visible", "kv_head_of", "reference_attention",
    "tiled_online_attention", "splitkv_partials", "merge_partials",
    "splitkv_attention", "split_bounds",
]


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head ``hq`` (contiguous groups of Hq/Hkv)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // (Hq // Hkv)


def visible_mask(rows, cols, Nq: int, Nk: int, causal: bool,
                 window=None) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: may query ``i`` attend to key ``j``.
    ``window``: None or (left, right), a negative bound meaning none."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    vis = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        vis &= cols[None, :] <= rows[:, None] + (Nk - Nq)
    if window is not None:
        left, right = window
        pos = rows[:, None] + (Nk - Nq)   # the query's place on the key axis
        if left >= 0:
            vis &= cols[None, :] >= pos - left
        if right >= 0:
            vis &= cols[None, :] <= pos + right
    return vis


def block_visible(rows, cols, block_mask_bh, block_size) -> np.ndarray:
    """Boolean [len(rows), len(cols)] of one head's block mask: block
    (i // bq, j // bk) non-zero."""
    bq, bk = block_size
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    bm = np.asarray(block_mask_bh) != 0
    return bm[(rows // bq)[:, None], (cols // bk)[None, :]]


def column_visible(rows, cols, col_bounds_b) -> np.ndarray:
    """Boolean [len(rows), len(cols)] of one sequence's column mask:
    ``col_bounds_b`` [Nk, 2] gives, per key column j, the query rows
    [lo_j, hi_j) that may see key j (an empty range hides the key)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    cb = np.asarray(col_bounds_b, dtype=np.int64)
    lo, hi = cb[cols, 0], cb[cols, 1]
    return (rows[:, None] >= lo[None, :]) & (rows[:, None] < hi[None, :])


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d or Hq % Hkv:
        raise ValueError("shape mismatch")
    return B, Hq, Hkv, Nq, Nk, d


def reference_attention(q, k, v, *, causal: bool, scale: float, rows=None,
                        return_sp: bool = False, window=None, block_mask=None,
                        block_size=(256, 64), col_bounds=None):
    """The definition, with S and P materialised per head in float64.

    S[i, j] = scale * sum_c q[i, c] k[j, c], set to -inf where key j is not
    visible to query i; P = row softmax of S; O = P V; lse[i] = logsumexp of
    row i of S.  ``rows`` restricts the computation to some query rows (the
    result then has ``len(rows)`` rows); ``return_sp`` also returns the
    per-head S and P arrays (shape [B, Hq, rows, Nk]).  ``window`` adds the
    sliding-window bounds (left, right) of ``visible_mask``; ``block_mask``
    ([B, Hq, nqb, nkb], broadcastable) keeps only the keys of non-zero
    blocks of ``block_size`` (query rows, keys).  ``col_bounds`` ([B, Nk, 2],
    one per sequence, shared by its heads) keeps key j only for the query
    rows lo_j <= i < hi_j (``column_visible``), on top of the other masks.
    """
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    vis = visible_mask(rows, np.arange(Nk), Nq, Nk, causal, window)
    O = np.zeros((B, Hq, R, d))
    lse = np.empty((B, Hq, R))
    if return_sp:
        S_all = np.empty((B, Hq, R, Nk))
        P_all = np.empty((B, Hq, R, Nk))
    if block_mask is not None:
        block_mask = np.broadcast_to(np.asarray(block_mask),
                                     (B, Hq) + np.shape(block_mask)[2:])
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h, rows] @ k[b, hk].T)
            vis_bh = vis
            if block_mask is not None:
                vis_bh = vis & block_visible(rows, np.arange(Nk),
                                             block_mask[b, h], block_size)
            if col_bounds is not None:
                vis_bh = vis_bh & column_visible(rows, np.arange(Nk),
                                                 col_bounds[b])
            S = np.where(vis_bh, S, -np.inf)
            m = S.max(axis=1)
            has = np.isfinite(m)
            m0 = np.where(has, m, 0.0)
            E = np.exp(S - m0[:, None])            # masked entries give 0
            den = E.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                P = np.where(has[:, None], E / np.where(has, den, 1.0)[:, None],
                             0.0)
                lse[b, h] = np.where(has, m0 + np.log(den), -np.inf)
            O[b, h] = P @ v[b, hk]
            if return_sp:
                S_all[b, h] = S
                P_all[b, h] = P
    if return_sp:
        return O, lse, S_all, P_all
    return O, lse


def tiled_online_attention(q, k, v, *, causal: bool, scale: float,
                           block_q: int, block_k: int):
    """The tiled online-softmax algorithm, in float64.

    For each Q block (``block_q`` rows, fixed) the K/V blocks (``block_k``
    keys) are visited in order; per row the running max ``m`` and running
    sum ``l`` are updated, the partial output is rescaled by
    ``exp(m - m_new)`` and gets ``P_ij V_j`` added; at the end ``O = O / l``
    and ``lse = m + ln l``.  Scale and mask are applied to each score block.
    Block sizes need not divide the sequence lengths.
    """
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be positive")
    O = np.zeros((B, Hq, Nq, d))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Nq, block_q):
                rows = np.arange(r0, min(r0 + block_q, Nq))
                Qi = q[b, h, rows]
                m = np.full(rows.size, -np.inf)
                l = np.zeros(rows.size)
                acc = np.zeros((rows.size, d))
                for c0 in range(0, Nk, block_k):
                    cols = np.arange(c0, min(c0 + block_k, Nk))
                    Sij = scale * (Qi @ k[b, hk, cols].T)
                    Sij = np.where(visible_mask(rows, cols, Nq, Nk, causal),
                                   Sij, -np.inf)
                    m_new = np.maximum(m, Sij.max(axis=1))
                    # rows with nothing visible yet keep a finite reference
                    ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    Pij = np.exp(Sij - ref[:, None])
                    alpha = np.exp(m - ref)
                    l = alpha * l + Pij.sum(axis=1)
                    acc = alpha[:, None] * acc + Pij @ v[b, hk, cols]
                    m = m_new
                with np.errstate(invalid="ignore", divide="ignore"):
                    has = l > 0
                    O[b, h, rows] = np.where(has[:, None],
                                             acc / np.where(has, l, 1.0)[:, None],
                                             0.0)
                    lse[b, h, rows] = np.where(has, m + np.log(l), -np.inf)
    return O, lse


def split_bounds(Nk: int, num_splits: int):
    """Contiguous key chunks [start, end) covering 0..Nk, sizes within 1."""
    if num_splits < 1:
        raise ValueError("num_splits must be positive")
    edges = np.linspace(0, Nk, num_splits + 1).round().astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:])]


def splitkv_partials(q, k, v, *, causal: bool, scale: float, bounds):
    """Per-chunk partial attention for the KV-split (Flash-Decoding) form.

    For each chunk ``[a, e)`` of keys and each query row: ``m_s`` = max of
    the visible scaled scores in the chunk (-inf if none), ``l_s`` = sum of
    exp(score - m_s) over them, and the unnormalised output
    ``Ot_s`` = sum of exp(score - m_s) * v_j.  Returns arrays shaped
    [S, B, Hq, Nq] (m, l) and [S, B, Hq, Nq, d] (Ot).
    """
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    S = len(bounds)
    m = np.full((S, B, Hq, Nq), -np.inf)
    l = np.zeros((S, B, Hq, Nq))
    Ot = np.zeros((S, B, Hq, Nq, d))
    rows = np.arange(Nq)
    for s, (a, e) in enumerate(bounds):
        if e <= a:
            continue
        cols = np.arange(a, e)
        vis = visible_mask(rows, cols, Nq, Nk, causal)
        for b in range(B):
            for h in range(Hq):
                hk = kv_head_of(h, Hq, Hkv)
                Sc = np.where(vis, scale * (q[b, h] @ k[b, hk, cols].T), -np.inf)
                ms = Sc.max(axis=1)
                ref = np.where(np.isfinite(ms), ms, 0.0)
                E = np.exp(Sc - ref[:, None])
                m[s, b, h] = ms
                l[s, b, h] = E.sum(axis=1)
                Ot[s, b, h] = E @ v[b, hk, cols]
    return m, l, Ot


def merge_partials(m, l, Ot):
    """Log-sum-exp merge of chunk partials, in chunk order.

    M = max_s m_s; w_s = exp(m_s - M) (0 for chunks with nothing visible);
    L = sum_s w_s l_s; O = sum_s w_s Ot_s / L; lse = M + ln L.
    """
    M = m.max(axis=0)
    ref = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(m - ref[None])                      # -inf chunks weigh 0
    L = (w * l).sum(axis=0)
    num = (w[..., None] * Ot).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        has = L > 0
        O = np.where(has[..., None], num / np.where(has, L, 1.0)[..., None], 0.0)
        lse = np.where(has, ref + np.log(L), -np.inf)
    return O, lse


def splitkv_attention(q, k, v, *, causal: bool, scale: float, num_splits=None,
                      bounds=None):
    """Split the keys into chunks, compute partials, merge them."""
    Nk = k.shape[2]
    if bounds is None:
        bounds = split_bounds(Nk, num_splits)
    return merge_partials(*splitkv_partials(q, k, v, causal=causal,
                                            scale=scale, bounds=bounds))
