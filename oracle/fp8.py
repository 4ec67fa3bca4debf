"""Plain CPU oracle for the attention forward on 8-bit floating-point inputs.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark import this module; the GPU library never
calls it and shares no code with it (numpy and the forward oracle only).

Sources: "FlashAttention-2 (KO)" (systems-analysis.info), section comparing
later versions: 8-bit floating point for extra speed; "FlashAttention
Analysis" (ryotta.opik.net), evolution by generation: FlashAttention-3
runs in FP8 low precision; the training-cost guide (tool.smithlab.co.kr),
version table (FP8 forward only) and FAQ (an FP8 forward is a
low-precision computation whose results differ from bf16).  The pages fix
neither the 8-bit format nor the scaling.  Readings taken:

* the format is OCP FP8 E4M3 (the gfx950 matrix cores' FP8): sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes
  subnormals m * 2^-9; S.1111.111 is NaN, there are no infinities; the
  largest finite magnitude is 448;
* per-block scaling is one fp32 "descale" factor per (batch, head) for each
  of Q, K and V: the real inputs are decode(code) * descale;
* V is stored transposed, [B, Hkv, d, Nk] (the key axis is the contraction
  axis of P V, and 8-bit matrix-core operands hold consecutive key values
  per lane).

The oracle is the forward definition on the decoded real inputs, in
float64: what the method computes exactly from those inputs.
"""
from __future__ import annotations

import numpy as np

from .attention import reference_attention

__all__ = ["decode_e4m3", "reference_attention_fp8"]


def decode_e4m3(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def reference_attention_fp8(q8, k8, vt8, q_descale, k_descale, v_descale, *,
                            causal: bool, scale: float, window=None):
    """q8 [B, Hq, Nq, d], k8 [B, Hkv, Nk, d], vt8 [B, Hkv, d, Nk] E4M3 codes;
    descales [B, Hq], [B, Hkv], [B, Hkv].  Returns (O, lse) of the forward
    definition on the real inputs decode(code) * descale."""
    q = decode_e4m3(q8) * np.asarray(q_descale, np.float64)[:, :, None, None]
    k = decode_e4m3(k8) * np.asarray(k_descale, np.float64)[:, :, None, None]
    vt = decode_e4m3(vt8) * np.asarray(v_descale, np.float64)[:, :, None, None]
    v = vt.transpose(0, 1, 3, 2)
    return reference_attention(q, k, v, causal=causal, scale=scale,
                               window=window)
