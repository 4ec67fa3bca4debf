"""Helpers for the GPU tests: device copies of the seeded bf16 inputs and
comparisons with the float64 oracle."""
from __future__ import annotations

import numpy as np

from fa_inputs import bf16_bits_to_f64

O_TOL = 1e-2     # max |O_gpu - O_oracle|
LSE_TOL = 1e-3   # max |lse_gpu - lse_oracle| over finite entries


def dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).to(device)


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def f64(bits):
    return bf16_bits_to_f64(bits)


def compare(O, lse, O_ref, lse_ref, o_tol=O_TOL, lse_tol=LSE_TOL, what=""):
    """Element-wise comparison; -inf lse entries must agree exactly and
    their O rows must be exactly 0.  Returns (max O err, max lse err)."""
    assert O.shape == O_ref.shape, (what, O.shape, O_ref.shape)
    assert lse.shape == lse_ref.shape, (what, lse.shape, lse_ref.shape)
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    ninf_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), ninf_ref,
                                  err_msg=f"{what}: -inf lse rows differ")
    if ninf_ref.any():
        assert np.all(O[ninf_ref] == 0.0), f"{what}: masked rows not zero"
    fin = ~ninf_ref
    eo = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    el = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    if eo > o_tol:
        idx = np.unravel_index(np.argmax(np.abs(O - O_ref)), O.shape)
        raise AssertionError(
            f"{what}: max |dO| = {eo:.3e} > {o_tol} at {tuple(map(int, idx))}: "
            f"got {O[idx]:.6f}, oracle {O_ref[idx]:.6f}")
    assert el <= lse_tol, f"{what}: max |dlse| = {el:.3e} > {lse_tol}"
    return eo, el


# Gradients: max |g - g_ref| <= GRAD_TOL * max |g_ref| + GRAD_ATOL per
# tensor.  Every gradient is a sum of products in which one factor (P or
# dS) was rounded to bf16 (relative error <= 2^-9) and D = dO . O uses the
# bf16 O; the relative bound is the O tolerance of the forward with the
# gradient's own scale in place of the unit scale of O.  The absolute term
# covers gradients that cancel to zero in exact arithmetic (a single key,
# uniform weights): dP - D is then the difference of two fp32 sums of
# terms below 100 in magnitude for unit-normal inputs (residue ~1e-6),
# times scale * |k| or |q|.
GRAD_TOL = 1e-2
GRAD_ATOL = 1e-5


def compare_grad(g, ref, tol=GRAD_TOL, atol=GRAD_ATOL, what=""):
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    if g.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(g - ref)))
    if err > tol * scale + atol:
        idx = np.unravel_index(np.argmax(np.abs(g - ref)), g.shape)
        raise AssertionError(
            f"{what}: max |err| = {err:.3e} > {tol} * {scale:.3e} + {atol} at "
            f"{tuple(map(int, idx))}: got {g[idx]:.6f}, oracle {ref[idx]:.6f}")
    return err / scale if scale > 0 else err


# FP8 forward: per-element tolerance derived from its arithmetic.  The
# kernel rounds each weight W_j to E4M3 (round to nearest even: an error
# uniform over one spacing of the E4M3 grid at W_j, 2^(floor(log2 W) - 3)
# for W >= 2^-6 and 2^-9 below), in a frame where the row's largest weight
# is at least 16, and normalises by the fp32 sum of the unrounded weights;
# the scores carry the 8-bit matrix cores' accumulation error (measured
# below 2^-13 of the sum of the magnitudes of the products; 2^-11 is
# used).  The rounding errors are independent and zero-mean, so the error
# of O_i,c is a sum of independent terms with standard deviation
#     sigma = sqrt(sum_j (spacing_j^2 / 12 + (dS_j W_j)^2) v_j,c^2) / sum_j W_j
# and the test allows 6 sigma (plus 1e-6 for fp32 sums).  lse is built from
# the unrounded weights: its error is bounded by the largest score error.
FP8_SIGMAS = 6.0
FP8_MFMA_REL = 2.0 ** -11


def e4m3_spacing(w):
    w = np.asarray(w, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(w, 2.0 ** -6)))
    return np.where(w >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)


def fp8_tolerance(P, v, dS):
    """P [R, Nk] row probabilities (oracle), v [Nk, d] real values, dS
    [R, Nk] bound on each score's error (natural-log units).  Returns the
    per-element tolerance [R, d] of O and the per-row bound [R] of lse."""
    pmax = P.max(axis=1, keepdims=True)
    W = np.where(pmax > 0, 16.0 * P / np.where(pmax > 0, pmax, 1.0), 0.0)
    var = np.where(W > 0, e4m3_spacing(W) ** 2 / 12.0 + (dS * W) ** 2, 0.0)
    sig = np.sqrt(var @ (v * v)) / np.maximum(W.sum(axis=1, keepdims=True),
                                               1e-300)
    lse_bound = np.where(P > 0, dS, 0.0).max(axis=1) + 1e-5
    return FP8_SIGMAS * sig + 1e-6, lse_bound
