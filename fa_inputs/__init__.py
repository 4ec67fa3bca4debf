"""Seeded synthetic inputs for the fused attention forward and backward, shared by the
oracle side and the GPU side.

This module holds no attention arithmetic.  It only

* names the five workloads (shapes, mask flag, scale, value distribution),
* draws the seeded fp32 values and rounds them to bf16 (round to nearest,
  ties to even), returning the raw bf16 bit patterns as ``uint16`` arrays,
* decodes bf16 bit patterns back to exact float values.

Layouts: Q is ``[B, Hq, Nq, d]``, K and V are ``[B, Hkv, Nk, d]``, all
contiguous with ``d`` fastest.

Generator recipe (one fresh ``numpy.random.default_rng(seed)`` per call):
draw Q, K, V in that order with ``standard_normal(dtype=float32)``; for the
outlier workload then draw the Q mask and the K mask as
``random() < 0.01`` (independent Bernoulli(0.01) per element) and multiply
the selected entries by 8 (a power of two, so exact before or after the
bf16 rounding); finally round every fp32 value to bf16.  The incoming
gradient dO of the backward pass is drawn N(0, 1) the same way from
``default_rng([seed, 0x64])``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_inputs", "make_qkv", "make_dout",
    "make_varlen", "VARLEN_PREFILL", "varlen_lengths", "make_paged",
    "f32_to_e4m3", "make_fp8", "sparse_block_mask",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, mask, scale, distribution."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    scale: float
    outliers: bool = False   # 1% of Q and K entries scaled by 8

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, in order: tiny, MHA d=64, causal d=128 with outlier
# scores, GQA prefill shaped like Qwen3-4B attention (32 query heads, 8 KV
# heads, head dim 128), and single-query split-KV decode over a 32K cache.
WORKLOADS = (
    Workload("tiny_b1_h1_n256_d64", 1, 1, 1, 256, 256, 64, False, 1.0 / 8.0),
    Workload("mha_b4_h16_n2048_d64", 4, 16, 16, 2048, 2048, 64, False,
             1.0 / math.sqrt(64)),
    Workload("causal_outlier_b2_h16_n4096_d128", 2, 16, 16, 4096, 4096, 128,
             True, 1.0 / math.sqrt(128), outliers=True),
    Workload("gqa_prefill_b1_hq32_hkv8_n8192_d128_causal", 1, 32, 8, 8192,
             8192, 128, True, 1.0 / math.sqrt(128)),
    Workload("decode_b16_hq32_hkv8_nq1_nk32768_d128", 16, 32, 8, 1, 32768,
             128, False, 1.0 / math.sqrt(128)),
)


def workload(i_or_name) -> Workload:
    if isinstance(i_or_name, int):
        return WORKLOADS[i_or_name]
    for w in WORKLOADS:
        if w.name == i_or_name:
            return w
    raise KeyError(i_or_name)


# ---------------------------------------------------------------- bf16 codec
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN maps to a quiet NaN (0x7FC0 with the sign kept); infinities and
    values that round past the largest finite bf16 become infinities.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        sign = (u >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)
        rounded = np.where(nan, sign | np.uint16(0x7FC0), rounded)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (no rounding happens)."""
    return bf16_bits_to_f32(b).astype(np.float64)


# ------------------------------------------------------------ the generator
def make_qkv(B, Hq, Hkv, Nq, Nk, d, *, seed=0, outliers=False,
             dist="normal", grid=None):
    """Draw Q, K, V as bf16 bit patterns (uint16 arrays).

    ``dist`` is ``"normal"`` (the recipe in the module docstring) or
    ``"grid"``: values drawn uniformly from the integers in
    ``[-grid, grid]`` times 1/8, which bf16 holds exactly; tests that need
    exactly representable shifted keys use it.
    """
    rng = np.random.default_rng(seed)
    shapes = ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d))
    if dist == "normal":
        q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in shapes)
    elif dist == "grid":
        g = 4 if grid is None else int(grid)
        q, k, v = (rng.integers(-g, g + 1, size=s).astype(np.float32) / 8.0
                   for s in shapes)
    else:
        raise ValueError(dist)
    if outliers:
        mq = rng.random(q.shape) < 0.01
        mk = rng.random(k.shape) < 0.01
        q = np.where(mq, q * np.float32(8.0), q).astype(np.float32)
        k = np.where(mk, k * np.float32(8.0), k).astype(np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_dout(B, Hq, Nq, d, *, seed=0):
    """The incoming gradient dO of the backward pass: i.i.d. N(0, 1) fp32
    cast to bf16 (bit patterns), from a stream of its own so that it is
    independent of Q, K, V drawn with the same seed."""
    rng = np.random.default_rng([seed, 0x64])
    return f32_to_bf16_bits(rng.standard_normal((B, Hq, Nq, d),
                                                dtype=np.float32))


def make_varlen(seqlens_q, seqlens_k, Hq, Hkv, d, *, seed=0):
    """A packed variable-length batch: sequence b has seqlens_q[b] query rows
    and seqlens_k[b] key/value rows.  Returns (q, k, v, cu_q, cu_k) with q
    [total_q, Hq, d], k and v [total_k, Hkv, d] as bf16 bit patterns
    (token-major, the rows of all sequences back to back) and the int32
    row offsets cu_q, cu_k (B + 1 entries, from 0).  The values are drawn
    like ``make_qkv``: N(0, 1) fp32 from ``default_rng(seed)`` (Q, then K,
    then V, each over the whole packed tensor), rounded to bf16."""
    seqlens_q = np.asarray(seqlens_q, dtype=np.int64)
    seqlens_k = np.asarray(seqlens_k, dtype=np.int64)
    if seqlens_q.shape != seqlens_k.shape or seqlens_q.ndim != 1:
        raise ValueError("one query and one key length per sequence")
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((int(cu_q[-1]), Hq, d), dtype=np.float32)
    k = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    v = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    return (f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v),
            cu_q, cu_k)


def make_paged(B, Hq, Hkv, Nq, d, page_size, max_pages, seqlens, *, seed=0,
               extra_pages=3):
    """A paged KV cache and queries: q [B, Hq, Nq, d] and the caches
    [num_pages, page_size, Hkv, d] as bf16 bit patterns, the int32 page
    table [B, max_pages] and the int32 lengths.  num_pages = B * max_pages
    + extra_pages; each sequence's pages are a seeded random draw without
    repeats from the pool, so pages are scattered and some pages belong to
    no sequence.  Values: N(0, 1) fp32 from ``default_rng(seed)`` (q, then
    the K cache, then the V cache), rounded to bf16; the page permutation
    comes from ``default_rng([seed, 0x70])``."""
    rng = np.random.default_rng(seed)
    num_pages = B * max_pages + extra_pages
    q = rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    kc = rng.standard_normal((num_pages, page_size, Hkv, d), dtype=np.float32)
    vc = rng.standard_normal((num_pages, page_size, Hkv, d), dtype=np.float32)
    perm = np.random.default_rng([seed, 0x70]).permutation(num_pages)
    table = perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    return (f32_to_bf16_bits(q), f32_to_bf16_bits(kc), f32_to_bf16_bits(vc),
            table, np.asarray(seqlens, dtype=np.int32))


def f32_to_e4m3(x) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 codes (uint8), round to nearest, ties to the
    even code; magnitudes that round above 448 are an error (the caller
    scales first).  Built by search over the 127 finite magnitudes, not by
    bit manipulation."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("non-finite input")
    codes = np.arange(127)                       # 0x00 .. 0x7E
    e, m = codes >> 3, codes & 7
    mags = np.where(e == 0, m / 512.0, (8 + m) * np.exp2(e - 10.0))
    a = np.abs(x)
    if np.any(a > 464.0) or np.any(a == 464.0):
        raise ValueError("magnitude rounds past 448")
    hi = np.clip(np.searchsorted(mags, a), 1, 126)
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    c = np.where(a >= mags[126], 126, np.where(pick_hi, hi, lo))
    c = np.where(a <= mags[0], 0, c)
    return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def make_fp8(B, Hq, Hkv, Nq, Nk, d, *, seed=0):
    """FP8 E4M3 inputs with one fp32 descale per (batch, head): the N(0, 1)
    fp32 draws of ``make_qkv`` (same generator and order), each head scaled
    by its own amax / 448 (rounded to fp32) and rounded to E4M3.  Returns
    (q8 [B, Hq, Nq, d], k8 [B, Hkv, Nk, d], vt8 [B, Hkv, d, Nk] -- V
    transposed --, q_descale [B, Hq], k_descale [B, Hkv], v_descale
    [B, Hkv])."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)

    def quant(x):
        amax = np.abs(x).reshape(x.shape[0], x.shape[1], -1).max(axis=2)
        ds = (np.maximum(amax, 1e-30) / 448.0).astype(np.float32)
        return f32_to_e4m3(x / ds[:, :, None, None].astype(np.float64)), ds
    q8, qd = quant(q)
    k8, kd = quant(k)
    v8, vd = quant(v)
    return q8, k8, np.ascontiguousarray(v8.transpose(0, 1, 3, 2)), qd, kd, vd


# A packed prefill batch of variable-length sequences, a serving mix: the
# heads of the GQA prefill workload, causal, each sequence its own prompt
# (query and key lengths equal); lengths drawn by ``varlen_lengths``.
VARLEN_PREFILL = dict(name="varlen_prefill_t32768_hq32_hkv8_d128_causal",
                      total=32768, lo=256, hi=8192, Hq=32, Hkv=8, d=128,
                      causal=True, scale=1.0 / math.sqrt(128))


def varlen_lengths(total, lo, hi, seed=0):
    """Sequence lengths that add up to ``total``: each drawn log-uniform in
    [lo, hi] (``exp(uniform(log lo, log hi))`` rounded to an integer, from
    ``default_rng([seed, 0x76])``), the last one cut to what is left."""
    rng = np.random.default_rng([seed, 0x76])
    out, left = [], int(total)
    while left > 0:
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = min(n, left)
        out.append(n)
        left -= n
    return out


def sparse_block_mask(Hq, Nq, Nk, density, *, seed=0, block=(128, 64)):
    """A block mask [1, Hq, ceil(Nq / 128), ceil(Nk / 64)] (uint8): each
    block kept with probability ``density`` (``default_rng([seed, 0x73])``,
    independent per head), plus, for every query block, the key blocks
    that hold the keys at its rows' own places (i + Nk - Nq), so that every
    row keeps its diagonal (local attention plus random blocks)."""
    bq, bk = block
    nqb, nkb = -(-Nq // bq), -(-Nk // bk)
    rng = np.random.default_rng([seed, 0x73])
    m = (rng.random((1, Hq, nqb, nkb)) < density).astype(np.uint8)
    for qb in range(nqb):
        lo = qb * bq + Nk - Nq
        hi = min((qb + 1) * bq, Nq) - 1 + Nk - Nq
        for kb in range(max(lo, 0) // bk, min(hi, Nk - 1) // bk + 1):
            m[:, :, qb, kb] = 1
    return m


def make_inputs(w, seed=0):
    """Q, K, V bit patterns for a workload (index, name or ``Workload``)."""
    if not isinstance(w, Workload):
        w = workload(w)
    return make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, seed=seed,
                    outliers=w.outliers)


def document_column_bounds(doc_lens, causal_docs=True):
    """Column bounds [N, 2] int32 of documents packed back to back in one
    sequence of N = sum(doc_lens) rows and keys: key j of the document
    [s, e) is seen by rows j .. e - 1 (causal inside the document) or
    s .. e - 1 (bidirectional)."""
    import numpy as np
    n = int(sum(doc_lens))
    out = np.empty((n, 2), dtype=np.int32)
    s = 0
    for L in doc_lens:
        e = s + int(L)
        j = np.arange(s, e)
        out[s:e, 0] = j if causal_docs else s
        out[s:e, 1] = e
        s = e
    return out


def prefix_lm_column_bounds(n, prefix):
    """Column bounds [n, 2] int32 of a prefix-LM mask: keys of the prefix
    seen by every row, later keys from their own row on."""
    import numpy as np
    j = np.arange(n)
    return np.stack([np.where(j < prefix, 0, j), np.full(n, n)],
                    axis=1).astype(np.int32)


def random_column_bounds(nq, nk, *, seed=0):
    """Column bounds [nk, 2] int32 with random row ranges inside [0, nq]
    (some empty)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    a = rng.integers(0, nq + 1, size=nk)
    b = rng.integers(0, nq + 1, size=nk)
    return np.stack([np.minimum(a, b), np.maximum(a, b)],
                    axis=1).astype(np.int32)


def random_doc_lens(total, lo, hi, *, seed=0):
    """Document lengths in [lo, hi] summing to ``total``."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out, left = [], total
    while left > 0:
        L = int(min(left, rng.integers(lo, hi + 1)))
        out.append(L)
        left -= L
    return out
