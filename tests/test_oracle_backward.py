"""CPU checks of the float64 backward oracle against facts it does not
compute itself: central finite differences of the forward definition, an
independent autograd implementation, invariants of the gradient, the
recomputation form against the definition, and planted mistakes that
these checks must catch."""
import math
import os
import types

import numpy as np
import pytest

from oracle import (recompute_backward, reference_attention,
                    reference_attention_backward)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "backward.py")


def _rand(B, Hq, Hkv, Nq, Nk, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, Hq, Nq, d))
    return q, k, v, do


def _numeric_grads(q, k, v, do, causal, scale, h=1e-5, window=None):
    """Central differences of L = sum(dO * O) with respect to every input
    element (the forward definition only)."""
    def loss(q_, k_, v_):
        O, _ = reference_attention(q_, k_, v_, causal=causal, scale=scale,
                                   window=window)
        return float((do * O).sum())
    grads = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros(arrs[which].shape)
        it = np.nditer(arrs[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = arrs[which][idx]
            arrs[which][idx] = x0 + h
            lp = loss(*arrs)
            arrs[which][idx] = x0 - h
            lm = loss(*arrs)
            arrs[which][idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


# B, Hq, Hkv, Nq, Nk, d, causal, scale
FD_CASES = [
    (1, 1, 1, 2, 2, 2, False, 0.7),
    (1, 2, 1, 3, 4, 3, False, 0.5),
    (1, 2, 1, 3, 4, 3, True, 0.5),     # bottom-right causal, Nq < Nk
    (2, 2, 2, 4, 4, 2, True, 1.1),
    (1, 4, 2, 3, 3, 3, True, 0.9),     # grouped-query heads
    (1, 1, 1, 5, 3, 2, True, 0.6),     # rows 0, 1 see no key
]


@pytest.mark.parametrize("case", FD_CASES, ids=str)
def test_definition_matches_finite_differences(case):
    B, Hq, Hkv, Nq, Nk, d, causal, scale = case
    q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=sum(case[:6]))
    dq, dk, dv = reference_attention_backward(q, k, v, do, causal=causal,
                                              scale=scale)
    nq, nk, nv = _numeric_grads(q, k, v, do, causal, scale)
    for got, want in ((dq, nq), (dk, nk), (dv, nv)):
        assert np.max(np.abs(got - want)) <= 1e-7 * (1 + np.max(np.abs(want)))


def test_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    for causal in (False, True):
        B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 9, 13, 8
        q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=7 + causal)
        scale = 0.3
        Q = torch.tensor(q, requires_grad=True)
        K = torch.tensor(k, requires_grad=True)
        V = torch.tensor(v, requires_grad=True)
        G = Hq // Hkv
        Kr, Vr = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
        S = scale * (Q @ Kr.transpose(-1, -2))
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nk)[None, :]
            S = S.masked_fill(j > i + (Nk - Nq), float("-inf"))
        O = torch.softmax(S, dim=-1) @ Vr
        O.backward(torch.tensor(do))
        dq, dk, dv = reference_attention_backward(q, k, v, do, causal=causal,
                                                  scale=scale)
        for got, want in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
            assert np.max(np.abs(got - want.numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (2, 3), (5, 4), (64, 64)])
def test_recompute_equals_definition(causal, bq, bk):
    q, k, v, do = _rand(1, 4, 2, 11, 17, 6, seed=bq * 10 + bk + causal)
    scale = 0.4
    O, lse = reference_attention(q, k, v, causal=causal, scale=scale)
    want = reference_attention_backward(q, k, v, do, causal=causal, scale=scale)
    got = recompute_backward(q, k, v, O, lse, do, causal=causal, scale=scale,
                             block_q=bq, block_k=bk)
    for g, w in zip(got, want):
        assert np.max(np.abs(g - w)) <= 1e-12


def test_recompute_with_rows_that_see_no_key():
    q, k, v, do = _rand(1, 2, 1, 7, 4, 3, seed=3)
    O, lse = reference_attention(q, k, v, causal=True, scale=0.5)
    assert np.isneginf(lse[0, 0, :3]).all()
    got = recompute_backward(q, k, v, O, lse, do, causal=True, scale=0.5,
                             block_q=2, block_k=3)
    want = reference_attention_backward(q, k, v, do, causal=True, scale=0.5)
    for g, w in zip(got, want):
        assert np.max(np.abs(g - w)) <= 1e-12
    assert np.all(got[0][0, :, :3] == 0)          # no gradient for those rows


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero(causal):
    """scale = 0: uniform weights over the visible keys, so dQ = dK = 0 and
    dV_j = sum over the rows that see key j of dO_i / (#keys row i sees)."""
    q, k, v, do = _rand(1, 2, 2, 6, 6, 4, seed=5)
    dq, dk, dv = reference_attention_backward(q, k, v, do, causal=causal,
                                              scale=0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    n = np.arange(1, 7) if causal else np.full(6, 6)
    want = np.zeros_like(dv)
    for i in range(6):
        for j in range(int(n[i])):
            want[0, :, j] += do[0, :, i] / n[i]
    assert np.max(np.abs(dv - want)) <= 1e-14


def test_key_shift_leaves_gradients_unchanged():
    """Adding one vector u to every key shifts each score row by a constant,
    which leaves P, O and so every gradient unchanged (the rows of dS sum to
    zero)."""
    q, k, v, do = _rand(1, 2, 1, 5, 7, 4, seed=9)
    u = np.random.default_rng(1).standard_normal(4)
    for causal in (False, True):
        a = reference_attention_backward(q, k, v, do, causal=causal, scale=0.5)
        b = reference_attention_backward(q, k + u, v, do, causal=causal,
                                         scale=0.5)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) <= 1e-12


def test_gqa_gradients_are_sums_over_the_group():
    q, k, v, do = _rand(1, 6, 2, 5, 8, 3, seed=12)
    G = 3
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        dq, dk, dv = reference_attention_backward(q, k, v, do, causal=causal,
                                                  scale=0.7)
        dq2, dk2, dv2 = reference_attention_backward(q, kr, vr, do,
                                                     causal=causal, scale=0.7)
        assert np.max(np.abs(dq - dq2)) <= 1e-14
        assert np.max(np.abs(dk - dk2.reshape(1, 2, G, 8, 3).sum(2))) <= 1e-14
        assert np.max(np.abs(dv - dv2.reshape(1, 2, G, 8, 3).sum(2))) <= 1e-14


MUTANTS = {
    "dropped_D": ("dS = Ph * (dP - D[:, None])", "dS = Ph * dP"),
    "dv_wrong_operand": ("dv[b, hk] += Ph.T @ do[b, h]",
                         "dv[b, hk] += Ph.T @ q[b, h]"),
    "dq_unscaled": ("dq[b, h] = scale * (dS @ k[b, hk])", "dq[b, h] = (dS @ k[b, hk])"),
    "dk_assigned": ("dk[b, hk] += scale * (dS.T @ q[b, h])",
                    "dk[b, hk] = scale * (dS.T @ q[b, h])"),
    "D_sign": ("D = (Ph * dP).sum(axis=1)", "D = -(Ph * dP).sum(axis=1)"),
    "recompute_lse_sign": ("np.exp(np.where(vis, S, 0.0) - Lr[:, None])",
                           "np.exp(np.where(vis, S, 0.0) + Lr[:, None])"),
    "recompute_D_from_v": ("D = (do * o).sum(axis=3)",
                           "D = (do * do).sum(axis=3)"),
}


def _load_mutant(old, new):
    src = open(_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_backward_mutant")
    exec(compile(src.replace(old, new), "oracle_backward_mutant", "exec"),
         mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_checks_catch_planted_mistake(name):
    mod = _load_mutant(*MUTANTS[name])
    caught = False
    for case in FD_CASES[1:5]:
        B, Hq, Hkv, Nq, Nk, d, causal, scale = case
        q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=sum(case[:6]))
        try:
            if name.startswith("recompute"):
                O, lse = reference_attention(q, k, v, causal=causal, scale=scale)
                got = mod.recompute_backward(q, k, v, O, lse, do, causal=causal,
                                             scale=scale, block_q=2, block_k=2)
            else:
                got = mod.reference_attention_backward(q, k, v, do,
                                                       causal=causal,
                                                       scale=scale)
            want = _numeric_grads(q, k, v, do, causal, scale)
            if any(np.max(np.abs(g - w)) > 1e-7 * (1 + np.max(np.abs(w)))
                   for g, w in zip(got, want)):
                caught = True
        except Exception:
            caught = True
        if caught:
            break
    assert caught, f"mutant {name} passed every check"


# ------------------------------------------------------- sliding window
# B, Hq, Hkv, Nq, Nk, d, causal, scale, window
WINDOW_FD_CASES = [
    (1, 2, 1, 4, 6, 2, False, 0.7, (1, 1)),
    (1, 2, 2, 5, 5, 3, True, 0.5, (2, -1)),
    (1, 1, 1, 6, 4, 2, False, 0.9, (0, 2)),    # Nq > Nk: empty rows
    (1, 4, 2, 3, 7, 2, False, 0.6, (-1, 0)),
]


@pytest.mark.parametrize("case", WINDOW_FD_CASES, ids=str)
def test_window_definition_matches_finite_differences(case):
    B, Hq, Hkv, Nq, Nk, d, causal, scale, window = case
    q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=sum(case[:6]) + 50)
    got = reference_attention_backward(q, k, v, do, causal=causal,
                                       scale=scale, window=window)
    want = _numeric_grads(q, k, v, do, causal, scale, window=window)
    for g, w in zip(got, want):
        assert np.max(np.abs(g - w)) <= 1e-7 * (1 + np.max(np.abs(w)))


def test_window_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Nq, Nk, d, scale = 1, 4, 2, 12, 15, 8, 0.3
    for window in ((3, 0), (2, 5), (-1, 1), (4, -1)):
        q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=60 + window[0])
        Q = torch.tensor(q, requires_grad=True)
        K = torch.tensor(k, requires_grad=True)
        V = torch.tensor(v, requires_grad=True)
        G = Hq // Hkv
        Kr, Vr = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
        S = scale * (Q @ Kr.transpose(-1, -2))
        c = torch.arange(Nq)[:, None] + (Nk - Nq)
        j = torch.arange(Nk)[None, :]
        hide = torch.zeros(Nq, Nk, dtype=torch.bool)
        if window[0] >= 0:
            hide |= j < c - window[0]
        if window[1] >= 0:
            hide |= j > c + window[1]
        O = torch.softmax(S.masked_fill(hide, float("-inf")), dim=-1) @ Vr
        O.backward(torch.tensor(do))
        got = reference_attention_backward(q, k, v, do, causal=False,
                                           scale=scale, window=window)
        for g, w in zip(got, (Q.grad, K.grad, V.grad)):
            assert np.max(np.abs(g - w.numpy())) <= 1e-12


def test_window_of_one_key_gradients():
    """window (0, 0): row i sees only key c = i + Nk - Nq with weight 1, so
    O_i = v_c does not depend on q or k (dQ = dK = 0) and dV_c = dO_i."""
    q, k, v, do = _rand(1, 2, 1, 5, 7, 3, seed=70)
    dq, dk, dv = reference_attention_backward(q, k, v, do, causal=False,
                                              scale=0.8, window=(0, 0))
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12
    want = np.zeros_like(dv)
    for h in range(2):
        for i in range(5):
            want[0, 0, i + 2] += do[0, h, i]
    assert np.max(np.abs(dv - want)) <= 1e-12


@pytest.mark.parametrize("window", [(2, 1), (0, -1), (5, 0)])
@pytest.mark.parametrize("bq,bk", [(1, 1), (3, 4), (64, 64)])
def test_window_recompute_equals_definition(window, bq, bk):
    q, k, v, do = _rand(1, 4, 2, 11, 17, 6, seed=bq + bk + window[0])
    scale = 0.4
    O, lse = reference_attention(q, k, v, causal=False, scale=scale,
                                 window=window)
    want = reference_attention_backward(q, k, v, do, causal=False,
                                        scale=scale, window=window)
    got = recompute_backward(q, k, v, O, lse, do, causal=False, scale=scale,
                             block_q=bq, block_k=bk, window=window)
    for g, w in zip(got, want):
        assert np.max(np.abs(g - w)) <= 1e-12


WINDOW_MUTANTS = {
    "window_dropped_in_definition": (
        "return_sp=True, window=window)", "return_sp=True)"),
    "window_dropped_in_recompute": (
        "visible_mask(rows, cols, Nq, Nk, causal, window)",
        "visible_mask(rows, cols, Nq, Nk, causal)"),
}


@pytest.mark.parametrize("name", list(WINDOW_MUTANTS))
def test_window_checks_catch_planted_mistake(name):
    mod = _load_mutant(*WINDOW_MUTANTS[name])
    B, Hq, Hkv, Nq, Nk, d, causal, scale, window = WINDOW_FD_CASES[0]
    q, k, v, do = _rand(B, Hq, Hkv, Nq, Nk, d, seed=sum(WINDOW_FD_CASES[0][:6]) + 50)
    if name.endswith("recompute"):
        O, lse = reference_attention(q, k, v, causal=causal, scale=scale,
                                     window=window)
        got = mod.recompute_backward(q, k, v, O, lse, do, causal=causal,
                                     scale=scale, block_q=2, block_k=2,
                                     window=window)
    else:
        got = mod.reference_attention_backward(q, k, v, do, causal=causal,
                                               scale=scale, window=window)
    want = _numeric_grads(q, k, v, do, causal, scale, window=window)
    assert any(np.max(np.abs(g - w)) > 1e-7 * (1 + np.max(np.abs(w)))
               for g, w in zip(got, want)), name
