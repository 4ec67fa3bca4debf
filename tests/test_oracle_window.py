"""CPU pins of the oracle's sliding-window mask: a closed form (a window of
one key), pure-Python brute force on tiny shapes, reductions to the causal
and unmasked cases, per-row key slices, and planted mistakes that these
pins must catch."""
import math
import os
import types

import numpy as np
import pytest

from oracle import reference_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

TOL = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _attn(mod=None):
    ref = reference_attention if mod is None else mod.reference_attention

    def f(q, k, v, causal, scale, window):
        return ref(q, k, v, causal=causal, scale=scale, window=window)
    return f


def pin_window_of_one_key(attn):
    """window (0, 0): query i sees only key c = i + Nk - Nq, so O_i = v_c and
    lse_i = scale q_i . k_c; a row whose c falls outside the keys sees
    nothing (O = 0, lse = -inf)."""
    rng = np.random.default_rng(40)
    for Nq, Nk in ((5, 7), (7, 5), (6, 6)):
        q, k, v = _rand(rng, 1, 2, Nq, 3), _rand(rng, 1, 1, Nk, 3), \
            _rand(rng, 1, 1, Nk, 3)
        O, lse = attn(q, k, v, False, 0.7, (0, 0))
        for h in range(2):
            for i in range(Nq):
                c = i + Nk - Nq
                if 0 <= c < Nk:
                    np.testing.assert_allclose(O[0, h, i], v[0, 0, c],
                                               rtol=0, atol=TOL)
                    assert abs(lse[0, h, i] - 0.7 * q[0, h, i] @ k[0, 0, c]) \
                        <= TOL
                else:
                    assert np.all(O[0, h, i] == 0) and lse[0, h, i] == -np.inf


def _brute(q, k, v, causal, scale, window):
    """Pure-Python loops: the visible keys of each row listed one by one."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    left, right = window
    O = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Nq):
                c = i + Nk - Nq
                keys = [j for j in range(Nk)
                        if (left < 0 or j >= c - left)
                        and (right < 0 or j <= c + right)
                        and (not causal or j <= c)]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = {j: scale * sum(q[b, h, i, t] * k[b, hk, j, t]
                                    for t in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                z = sum(w.values())
                lse[b, h, i] = mx + math.log(z)
                for t in range(d):
                    O[b, h, i, t] = sum(w[j] * v[b, hk, j, t] for j in keys) / z
    return O, lse


def pin_window_brute_force(attn):
    """Every window bound in {-1, 0, 1, 2} on each side, with and without
    the causal flag, Nq < Nk, Nq = Nk and Nq > Nk, GQA 2:1."""
    rng = np.random.default_rng(41)
    for Nq, Nk in ((3, 5), (4, 4), (5, 3)):
        q, k, v = _rand(rng, 1, 2, Nq, 2), _rand(rng, 1, 1, Nk, 2), \
            _rand(rng, 1, 1, Nk, 2)
        for left in (-1, 0, 1, 2):
            for right in (-1, 0, 1, 2):
                for causal in (False, True):
                    O, lse = attn(q, k, v, causal, 0.9, (left, right))
                    Ob, lb = _brute(q, k, v, causal, 0.9, (left, right))
                    np.testing.assert_allclose(O, Ob, rtol=0, atol=TOL)
                    fin = np.isfinite(lb)
                    np.testing.assert_array_equal(np.isfinite(lse), fin)
                    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0,
                                               atol=TOL)


def pin_window_reductions(attn):
    """(-1, 0) and a left bound past every key with right 0 give the causal
    mask; bounds past every key on both sides (or none) give no mask.  The
    causal and unmasked forms are the oracle's own, pinned elsewhere."""
    rng = np.random.default_rng(42)
    for Nq, Nk in ((9, 13), (13, 9)):
        q, k, v = _rand(rng, 1, 2, Nq, 4), _rand(rng, 1, 2, Nk, 4), \
            _rand(rng, 1, 2, Nk, 4)
        Oc, lc = reference_attention(q, k, v, causal=True, scale=0.5)
        Of, lf = reference_attention(q, k, v, causal=False, scale=0.5)
        for w, (Oe, le) in (((-1, 0), (Oc, lc)), ((Nk + Nq, 0), (Oc, lc)),
                            ((-1, -1), (Of, lf)),
                            ((Nk + Nq, Nk + Nq), (Of, lf))):
            O, lse = attn(q, k, v, False, 0.5, w)
            np.testing.assert_array_equal(O, Oe)
            np.testing.assert_array_equal(lse, le)
        # the window is intersected with the causal flag
        O, lse = attn(q, k, v, True, 0.5, (-1, 3))
        np.testing.assert_array_equal(O, Oc)


def pin_window_key_slices(attn):
    """Row by row, the windowed result equals unmasked attention over the
    row's own slice of keys [c - left, c + right] (cut to the keys)."""
    rng = np.random.default_rng(43)
    Nq, Nk, left, right = 40, 50, 7, 3
    q, k, v = _rand(rng, 1, 1, Nq, 8), _rand(rng, 1, 1, Nk, 8), \
        _rand(rng, 1, 1, Nk, 8)
    O, lse = attn(q, k, v, False, 0.3, (left, right))
    for i in range(Nq):
        c = i + Nk - Nq
        a, e = max(c - left, 0), min(c + right, Nk - 1) + 1
        Oi, li = reference_attention(q[:, :, i:i + 1], k[:, :, a:e],
                                     v[:, :, a:e], causal=False, scale=0.3)
        np.testing.assert_allclose(O[0, 0, i], Oi[0, 0, 0], rtol=0, atol=TOL)
        assert abs(lse[0, 0, i] - li[0, 0, 0]) <= TOL


WINDOW_PINS = [pin_window_of_one_key, pin_window_brute_force,
               pin_window_reductions, pin_window_key_slices]


@pytest.mark.parametrize("pin", WINDOW_PINS, ids=lambda p: p.__name__)
def test_window_pins(pin):
    pin(_attn())


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "attention.py")

MUTANTS = {
    "left_off_by_one": ("vis &= cols[None, :] >= pos - left",
                        "vis &= cols[None, :] > pos - left"),
    "right_off_by_one": ("vis &= cols[None, :] <= pos + right",
                         "vis &= cols[None, :] < pos + right"),
    "top_left_window": ("pos = rows[:, None] + (Nk - Nq)",
                        "pos = rows[:, None]"),
    "bounds_swapped": ("vis &= cols[None, :] >= pos - left",
                       "vis &= cols[None, :] >= pos - right"),
    "window_replaces_causal": ("    if window is not None:\n        left, right = window",
                               "    if window is not None:\n        vis[:] = True\n        left, right = window"),
    "window_ignored": ("    if window is not None:\n        left, right = window",
                       "    if False:\n        left, right = window"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_window_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in WINDOW_PINS:
        try:
            pin(_attn(mod))
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no window pin caught the planted mistake {name}"
