"""Work and traffic counts used to report throughput, and the MI355X peaks.

The FLOP count follows the training-cost guide (tool.smithlab.co.kr,
"attention compute and training cost" section): a causal attention forward
costs 2 * N * h * d FLOPs per token per layer, i.e. two N x N x d products
of 2 FLOPs per multiply-add, halved by the causal mask.  For a batch this is
4 * B * Hq * Nq * Nk * d, halved when causal.
"""
from __future__ import annotations

# MI355X published peaks (dense, no structured sparsity).
PEAK_BF16_MFMA_TFLOPS = 2500.0     # bf16 / fp16 dense matrix-core peak
PEAK_FP8_MFMA_TFLOPS = 5000.0      # fp8 dense matrix-core peak
PEAK_HBM_GBS = 8000.0              # HBM3E bandwidth
PEAK_FP32_VECTOR_TFLOPS = 157.3


def attention_fwd_flops(B, Hq, Nq, Nk, d, causal) -> float:
    """Forward FLOPs: QK^T and PV, 2 FLOPs per multiply-add; /2 if causal."""
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2.0 if causal else f


def visible_pairs(Nq, Nk, causal, window=None) -> int:
    """Exact number of visible (query row, key) pairs of one head: row i,
    placed at c = i + Nk - Nq, sees keys max(0, c - left) .. min(Nk - 1,
    c + right) (right capped at 0 when causal; -1 is no bound)."""
    import numpy as np
    left, right = (-1, -1) if window is None else window
    c = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    lo = np.zeros(Nq, dtype=np.int64) if left < 0 else np.maximum(0, c - left)
    hi = np.full(Nq, Nk - 1, dtype=np.int64) if right < 0 else \
        np.minimum(Nk - 1, c + right)
    if causal:
        hi = np.minimum(hi, c)
    return int(np.maximum(hi - lo + 1, 0).sum())


def visible_keys(Nq, Nk, causal, window=None) -> int:
    """Keys that at least one query row sees (the K/V rows a windowed call
    must read): the union of the rows' key ranges, which is one range."""
    left, right = (-1, -1) if window is None else window
    c0, c1 = Nk - Nq, Nk - 1           # places of the first and last rows
    lo = 0 if left < 0 else max(0, c0 - left)
    hi = Nk - 1 if right < 0 else min(Nk - 1, c1 + right)
    if causal:
        hi = min(hi, c1)
    return max(hi - lo + 1, 0)


def block_pair_counts(Nq, Nk, causal, block_size):
    """Visible (query row, key) pairs inside each (query block, key block)
    of a block mask's grid: an array [ceil(Nq / bq), ceil(Nk / bk)]."""
    import numpy as np
    bq, bk = block_size
    nqb, nkb = -(-Nq // bq), -(-Nk // bk)
    c = np.arange(Nq, dtype=np.int64) + (Nk - Nq)       # each row's place
    hi = np.minimum(c, Nk - 1) if causal else np.full(Nq, Nk - 1)
    k0 = np.arange(nkb, dtype=np.int64) * bk
    k1 = np.minimum(k0 + bk, Nk) - 1
    per_row = np.clip(np.minimum(hi[:, None], k1[None, :]) - k0[None, :] + 1,
                      0, None)                           # [Nq, nkb]
    out = np.zeros((nqb, nkb), dtype=np.int64)
    np.add.at(out, np.arange(Nq) // bq, per_row)
    return out


def column_mask_pairs(bounds, Nq, Nk, causal) -> int:
    """Visible (query row, key) pairs of one head under a column-interval
    mask: key j (``bounds[j] = (lo, hi)``) is seen by rows lo .. hi - 1,
    from its causal place j - (Nk - Nq) on when causal."""
    import numpy as np
    b = np.asarray(bounds, dtype=np.int64)
    lo = np.maximum(b[:, 0], 0)
    if causal:
        lo = np.maximum(lo, np.arange(Nk, dtype=np.int64) - (Nk - Nq))
    hi = np.minimum(b[:, 1], Nq)
    return int(np.maximum(hi - lo, 0).sum())


def attention_window_flops(B, Hq, Nq, Nk, d, causal, window) -> float:
    """Forward FLOPs of a windowed mask: 4 d per visible pair (the two
    products), counted exactly."""
    return 4.0 * B * Hq * d * visible_pairs(Nq, Nk, causal, window)


def attention_bwd_flops(B, Hq, Nq, Nk, d, causal) -> float:
    """Backward FLOPs: the five N x N x d products of the recomputation
    form (scores, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q), i.e.
    2.5 times the forward, the factor the training-cost guide gives; /2 if
    causal.  Products an implementation repeats are not counted."""
    return 2.5 * attention_fwd_flops(B, Hq, Nq, Nk, d, causal)


def attention_fwd_bytes(B, Hq, Hkv, Nq, Nk, d, out_bytes=2, in_bytes=2) -> float:
    """Algorithmic HBM bytes: Q, K, V read once, O and the fp32 lse written
    once.  Re-reads of K/V by several Q blocks and split-KV partials are an
    implementation's overhead and are not counted."""
    q = B * Hq * Nq * d * in_bytes
    kv = 2 * B * Hkv * Nk * d * in_bytes
    o = B * Hq * Nq * d * out_bytes
    lse = B * Hq * Nq * 4
    return float(q + kv + o + lse)


def lse_bytes(B, Hq, Nq) -> int:
    """Bytes of the saved per-row statistic: one fp32 per query row."""
    return 4 * B * Hq * Nq


def training_attention_flops_per_token(seq_len, heads, head_dim, layers,
                                       backward_factor=2.5) -> float:
    """Causal training FLOPs per token: forward plus a backward priced at
    ``backward_factor`` times the forward (recomputation included)."""
    fwd_per_token = attention_fwd_flops(1, heads, seq_len, seq_len, head_dim,
                                        True) / seq_len
    return (1.0 + backward_factor) * fwd_per_token * layers
