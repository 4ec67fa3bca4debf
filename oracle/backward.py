"""Plain float64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark import this module.  The GPU library never
calls it, and it shares no code with the GPU path: it imports numpy and the
forward oracle of this package only.

The quantity is the gradient of the forward result O = softmax(scale * Q K^T
+ mask) V with respect to Q, K and V, for an incoming gradient dO of the same
shape as O (equivalently: of the scalar sum(dO * O)).  Layouts as in the
forward oracle:

    q, do, dq : [B, Hq, Nq, d]        k, v, dk, dv : [B, Hkv, Nk, d]

Sources (pages are named by title; sections as printed on them):

* "FlashAttention Analysis" (ryotta.opik.net), section 4 "Recomputation":
  the backward pass needs the attention probabilities, which are not
  stored; it recomputes S and P on chip from Q, K and the per-row statistics
  kept by the forward pass.
* FlashAttention version / GPU / training-cost guide (tool.smithlab.co.kr),
  section on attention memory during training: the forward pass keeps one
  fp32 logsumexp per query row for the backward pass; section on attention
  compute: the backward pass costs 2.5 times the forward FLOPs.

The gradient itself is the chain rule through the three steps of the
definition (S = scale Q K^T with the mask, P = row softmax of S, O = P V):

    dV = P^T dO                      dP = dO V^T
    dS = P * (dP - D),  D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
    dQ = scale dS K                  dK = scale dS^T Q

and with grouped-query attention each KV head receives the sum of the
gradients of all the query heads that read it.  Masked entries have P = 0
and so no gradient.  A query row that sees no key (O = 0, lse = -inf) gives
no gradient either.  ``window`` is the forward oracle's sliding window
(left, right); it only changes which entries are masked.
"""
from __future__ import annotations

import numpy as np

from .attention import _check, kv_head_of, reference_attention, visible_mask

__all__ = ["reference_attention_backward", "recompute_backward"]


def reference_attention_backward(q, k, v, do, *, causal: bool, scale: float,
                                 window=None):
    """The gradients from the definition, with S, P, dP and dS materialised
    per head in float64.  Returns (dq, dk, dv)."""
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    _, _, _, P = reference_attention(q, k, v, causal=causal, scale=scale,
                                     return_sp=True, window=window)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            Ph = P[b, h]                                  # [Nq, Nk]
            dv[b, hk] += Ph.T @ do[b, h]
            dP = do[b, h] @ v[b, hk].T                    # [Nq, Nk]
            D = (Ph * dP).sum(axis=1)                     # [Nq]
            dS = Ph * (dP - D[:, None])
            dq[b, h] = scale * (dS @ k[b, hk])
            dk[b, hk] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def recompute_backward(q, k, v, o, lse, do, *, causal: bool, scale: float,
                       block_q: int, block_k: int, window=None):
    """The recomputation form, block by block, in float64.

    D_i = dO_i . O_i is formed once per row from the forward output.  Then
    for every pair of a Q block (``block_q`` rows) and a K/V block
    (``block_k`` keys) the scores are recomputed, P = exp(S - lse) from the
    saved per-row statistic, and the block's contributions
    dV += P^T dO, dP = dO V^T, dS = P (dP - D), dQ += scale dS K,
    dK += scale dS^T Q are accumulated.  Block sizes need not divide the
    sequence lengths.  Returns (dq, dk, dv)."""
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be positive")
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    D = (do * o).sum(axis=3)                              # [B, Hq, Nq]
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Nq, block_q):
                rows = np.arange(r0, min(r0 + block_q, Nq))
                L = lse[b, h, rows]
                has = np.isfinite(L)
                Lr = np.where(has, L, 0.0)
                for c0 in range(0, Nk, block_k):
                    cols = np.arange(c0, min(c0 + block_k, Nk))
                    S = scale * (q[b, h, rows] @ k[b, hk, cols].T)
                    vis = visible_mask(rows, cols, Nq, Nk, causal, window)
                    vis &= has[:, None]
                    P = np.where(vis, np.exp(np.where(vis, S, 0.0) - Lr[:, None]),
                                 0.0)
                    dv[b, hk, cols] += P.T @ do[b, h, rows]
                    dP = do[b, h, rows] @ v[b, hk, cols].T
                    dS = P * (dP - D[b, h, rows][:, None])
                    dq[b, h, rows] += scale * (dS @ k[b, hk, cols])
                    dk[b, hk, cols] += scale * (dS.T @ q[b, h, rows])
    return dq, dk, dv
