"""CPU checks of the float64 oracle against facts it does not compute itself:
hand-worked examples, closed forms, invariants, pure-Python brute force,
an independent library implementation, and planted mistakes that the pins
must catch."""
import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest

from oracle import (reference_attention, tiled_online_attention,
                    splitkv_attention, splitkv_partials, merge_partials,
                    split_bounds, visible_mask)
import oracle.attention as oracle_attention
from tests.oracle_pins import ALL_PINS

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _ref(q, k, v, causal, scale):
    return reference_attention(q, k, v, causal=causal, scale=scale)


def _tiled(bq, bk):
    def f(q, k, v, causal, scale):
        return tiled_online_attention(q, k, v, causal=causal, scale=scale,
                                      block_q=bq, block_k=bk)
    return f


def _split(s):
    def f(q, k, v, causal, scale):
        return splitkv_attention(q, k, v, causal=causal, scale=scale,
                                 num_splits=min(s, k.shape[2]))
    return f


FORMS = {
    "definition": _ref,
    "tiled_1x1": _tiled(1, 1),
    "tiled_2x3": _tiled(2, 3),
    "tiled_big": _tiled(64, 64),
    "split_2": _split(2),
    "split_3": _split(3),
}


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pins(form, pin):
    pin(FORMS[form])


# --------------------------------------------------- independent library
def test_matches_torch_sdpa_float64():
    """torch's scaled_dot_product_attention (CPU, float64) is an
    independent implementation of the same definition; logsumexp is taken
    with torch.logsumexp over torch-computed masked scores."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(11)
    cases = [  # B, Hq, Hkv, Nq, Nk, d, causal
        (2, 4, 4, 17, 17, 8, False),
        (1, 8, 2, 33, 33, 16, True),
        (2, 4, 1, 5, 29, 8, True),     # bottom-right alignment, Nq < Nk
        (1, 2, 2, 1, 40, 4, False),    # single query (decode)
    ]
    for B, Hq, Hkv, Nq, Nk, d, causal in cases:
        q = rng.standard_normal((B, Hq, Nq, d))
        k = rng.standard_normal((B, Hkv, Nk, d))
        v = rng.standard_normal((B, Hkv, Nk, d))
        scale = 1.0 / math.sqrt(d)
        O, lse = reference_attention(q, k, v, causal=causal, scale=scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq) \
            if causal else None
        To = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                            scale=scale, enable_gqa=True)
        np.testing.assert_allclose(O, To.numpy(), rtol=0, atol=1e-12)
        kr = tk.repeat_interleave(Hq // Hkv, dim=1)
        s = scale * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            s = s.masked_fill(~mask, float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(),
                                   rtol=0, atol=1e-12)


def test_matches_scipy_softmax_rows():
    """Rows of P equal scipy's softmax of the masked scaled scores, and
    lse equals scipy's logsumexp of the same row."""
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 6, 5))
    k = rng.standard_normal((1, 1, 6, 5))
    v = rng.standard_normal((1, 1, 6, 5))
    O, lse, S, P = reference_attention(q, k, v, causal=True, scale=0.5,
                                       return_sp=True)
    for i in range(6):
        row = 0.5 * np.array([q[0, 0, i] @ k[0, 0, j] for j in range(i + 1)])
        np.testing.assert_allclose(P[0, 0, i, :i + 1], softmax(row), atol=1e-14)
        assert np.all(P[0, 0, i, i + 1:] == 0.0)
        np.testing.assert_allclose(lse[0, 0, i], logsumexp(row), atol=1e-14)


# --------------------------------------------------- algebra of the method
def test_rows_of_p_sum_to_one():
    rng = np.random.default_rng(13)
    for causal in (False, True):
        q, k, v = (rng.standard_normal((2, 3, 11, 4)) * 3 for _ in range(3))
        _, _, S, P = reference_attention(q, k, v, causal=causal, scale=1.0,
                                         return_sp=True)
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-12)
        vis = visible_mask(np.arange(11), np.arange(11), 11, 11, causal)
        assert np.all(P[..., ~vis] == 0.0)
        assert np.all(np.isneginf(S[..., ~vis]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (3, 5), (16, 16), (40, 40), (7, 13),
                                   (64, 3)])
@pytest.mark.parametrize("nq,nk", [(40, 40), (13, 37)])
def test_tiled_online_equals_definition(causal, bq, bk, nq, nk):
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 4, nq, 8)) * 2
    k = rng.standard_normal((1, 2, nk, 8)) * 2
    v = rng.standard_normal((1, 2, nk, 8))
    O0, l0 = reference_attention(q, k, v, causal=causal, scale=0.35)
    O1, l1 = tiled_online_attention(q, k, v, causal=causal, scale=0.35,
                                    block_q=bq, block_k=bk)
    np.testing.assert_allclose(O1, O0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l0, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 2, 7, 37])
def test_split_merge_equals_definition(causal, splits):
    rng = np.random.default_rng(15)
    q = rng.standard_normal((2, 4, 13, 8)) * 2
    k = rng.standard_normal((2, 1, 37, 8)) * 2
    v = rng.standard_normal((2, 1, 37, 8))
    O0, l0 = reference_attention(q, k, v, causal=causal, scale=0.4)
    O1, l1 = splitkv_attention(q, k, v, causal=causal, scale=0.4,
                               num_splits=splits)
    np.testing.assert_allclose(O1, O0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l0, atol=1e-12, rtol=0)


def test_split_with_empty_and_fully_masked_chunks():
    """Chunks with no key, and chunks whose keys are all hidden by the
    causal mask, weigh nothing in the merge."""
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 4, 6))
    k = rng.standard_normal((1, 2, 20, 6))
    v = rng.standard_normal((1, 2, 20, 6))
    bounds = [(0, 0), (0, 5), (5, 5), (5, 17), (17, 20)]  # Nq=4: row 0 sees 0..16
    O0, l0 = reference_attention(q, k, v, causal=True, scale=0.5)
    m, l, Ot = splitkv_partials(q, k, v, causal=True, scale=0.5, bounds=bounds)
    assert np.all(np.isneginf(m[0])) and np.all(l[0] == 0)
    assert np.isneginf(m[4, 0, 0, 0])            # row 0 sees nothing in 17..19
    O1, l1 = merge_partials(m, l, Ot)
    np.testing.assert_allclose(O1, O0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l0, atol=1e-12, rtol=0)


def test_split_bounds_cover_keys():
    for nk in (1, 5, 37, 32768):
        for s in (1, 2, 7, 16):
            b = split_bounds(nk, s)
            assert b[0][0] == 0 and b[-1][1] == nk and len(b) == s
            assert all(x[1] == y[0] for x, y in zip(b, b[1:]))
            sizes = [e - a for a, e in b]
            assert max(sizes) - min(sizes) <= 1


def test_row_subset_matches_full():
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((1, 2, 19, 4)) for _ in range(3))
    O, lse = reference_attention(q, k, v, causal=True, scale=0.5)
    rows = [0, 5, 18]
    Os, ls = reference_attention(q, k, v, causal=True, scale=0.5, rows=rows)
    np.testing.assert_array_equal(Os, O[:, :, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])


# ------------------------------------------------------- planted mistakes
_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "attention.py")

MUTANTS = {
    "dropped_scale": ("S = scale * (q[b, h, rows] @ k[b, hk].T)",
                      "S = (q[b, h, rows] @ k[b, hk].T)"),
    "v_replaced_by_k": ("O[b, h] = P @ v[b, hk]", "O[b, h] = P @ k[b, hk]"),
    "lse_sign": ("m0 + np.log(den)", "m0 - np.log(den)"),
    "no_max_subtraction": ("E = np.exp(S - m0[:, None])", "E = np.exp(S)"),
    "interleaved_gqa": ("return hq // (Hq // Hkv)", "return hq % Hkv"),
    "top_left_causal": ("cols[None, :] <= rows[:, None] + (Nk - Nq)",
                        "cols[None, :] <= rows[:, None]"),
    "causal_off_by_one": ("cols[None, :] <= rows[:, None] + (Nk - Nq)",
                          "cols[None, :] < rows[:, None] + (Nk - Nq)"),
    "unnormalised": ("P = np.where(has[:, None], E / np.where(has, den, 1.0)[:, None],",
                     "P = np.where(has[:, None], E,"),
    "tiled_no_rescale_acc": ("acc = alpha[:, None] * acc + Pij @ v[b, hk, cols]",
                             "acc = acc + Pij @ v[b, hk, cols]"),
    "tiled_no_rescale_l": ("l = alpha * l + Pij.sum(axis=1)",
                           "l = l + Pij.sum(axis=1)"),
    "tiled_stale_max": ("m = m_new\n", "m = m\n"),
    "merge_weight_sign": ("w = np.exp(m - ref[None])", "w = np.exp(ref[None] - m)"),
    "merge_no_weight_on_l": ("L = (w * l).sum(axis=0)", "L = l.sum(axis=0)"),
}


def _load_mutant(old, new):
    src = open(_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _load_mutant(*MUTANTS[name])
    if name.startswith("tiled"):
        def attn(q, k, v, causal, scale):
            return mod.tiled_online_attention(q, k, v, causal=causal,
                                              scale=scale, block_q=2, block_k=2)
    elif name.startswith("merge"):
        def attn(q, k, v, causal, scale):
            return mod.splitkv_attention(q, k, v, causal=causal, scale=scale,
                                         num_splits=min(3, k.shape[2]))
    else:
        def attn(q, k, v, causal, scale):
            return mod.reference_attention(q, k, v, causal=causal, scale=scale)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(attn)
        except Exception as e:  # an assertion, or a crash in the mutant
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
