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
