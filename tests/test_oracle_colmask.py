"""CPU pins of the column-interval mask of the forward oracle (per key
column j, the query rows lo_j <= i < hi_j may see key j): the intervals
that reproduce the causal mask and the sliding window, document
(block-diagonal) masks against per-document slices, keys hidden from every
row against the oracle without them, brute force in pure Python on random
intervals, a row that sees nothing, and planted mistakes these pins catch."""
import math
import os
import types

import numpy as np
import pytest

from oracle import reference_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _qkv(seed, B=2, Hq=4, Hkv=2, Nq=9, Nk=9, d=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, Nq, d)),
            rng.standard_normal((B, Hkv, Nk, d)),
            rng.standard_normal((B, Hkv, Nk, d)))


def _bounds(B, lo, hi):
    cb = np.stack([np.asarray(lo), np.asarray(hi)], axis=-1)
    return np.broadcast_to(cb, (B,) + cb.shape).copy()


def pin_intervals_make_causal(ref):
    """Key j seen by the rows i with j <= i + Nk - Nq: lo_j = j - (Nk - Nq)
    (at least 0), hi_j = Nq."""
    for Nq, Nk in ((9, 9), (5, 9)):
        q, k, v = _qkv(1, Nq=Nq, Nk=Nk)
        j = np.arange(Nk)
        cb = _bounds(2, np.maximum(j - (Nk - Nq), 0), np.full(Nk, Nq))
        O, L = ref(q, k, v, causal=False, scale=0.5, col_bounds=cb)
        Or, Lr = reference_attention(q, k, v, causal=True, scale=0.5)
        np.testing.assert_allclose(O, Or, atol=1e-12)
        np.testing.assert_allclose(L, Lr, atol=1e-12)


def pin_intervals_make_window(ref):
    """Causal with a 2-key left window: key j seen by rows j - off .. j -
    off + 2."""
    q, k, v = _qkv(2, Nq=7, Nk=10)
    off = 3
    j = np.arange(10)
    cb = _bounds(2, np.clip(j - off, 0, 7), np.clip(j - off + 3, 0, 7))
    O, L = ref(q, k, v, causal=True, scale=0.4, col_bounds=cb)
    Or, Lr = reference_attention(q, k, v, causal=True, scale=0.4,
                                 window=(2, 0))
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(L, Lr, atol=1e-12)


def pin_documents_are_slices(ref):
    """Documents [0, 4) and [4, 9) packed in one sequence: each key is seen
    by its own document's rows only, so each document's rows equal the
    oracle on that document's slice (bidirectional, and causal)."""
    q, k, v = _qkv(3)
    doc = np.array([0] * 4 + [1] * 5)
    start = np.where(doc == 0, 0, 4)
    end = np.where(doc == 0, 4, 9)
    for causal in (False, True):
        lo = np.arange(9) if causal else start
        cb = _bounds(2, lo, end)
        O, L = ref(q, k, v, causal=False, scale=0.3, col_bounds=cb)
        for s, e in ((0, 4), (4, 9)):
            Or, Lr = reference_attention(q[:, :, s:e], k[:, :, s:e],
                                         v[:, :, s:e], causal=causal,
                                         scale=0.3)
            np.testing.assert_allclose(O[:, :, s:e], Or, atol=1e-12)
            np.testing.assert_allclose(L[:, :, s:e], Lr, atol=1e-12)


def pin_hidden_keys_drop_out(ref):
    """Keys with an empty row range are never seen: the oracle on the
    remaining keys; keys seen by every row leave nothing to mask."""
    q, k, v = _qkv(4)
    lo = np.zeros(9, dtype=np.int64)
    hi = np.full(9, 9)
    O0, L0 = ref(q, k, v, causal=False, scale=0.7, col_bounds=_bounds(2, lo, hi))
    Or, Lr = reference_attention(q, k, v, causal=False, scale=0.7)
    np.testing.assert_array_equal(O0, Or)
    np.testing.assert_array_equal(L0, Lr)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 1, 1], dtype=bool)
    O, L = ref(q, k, v, causal=False, scale=0.7,
               col_bounds=_bounds(2, np.where(keep, 0, 5), np.where(keep, 9, 5)))
    Or, Lr = reference_attention(q, k[:, :, keep], v[:, :, keep],
                                 causal=False, scale=0.7)
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(L, Lr, atol=1e-12)


def pin_brute_force(ref):
    """Random intervals against softmax over the visible keys, in pure
    Python."""
    rng = np.random.default_rng(5)
    q, k, v = _qkv(5, B=1, Hq=2, Hkv=1, Nq=5, Nk=6, d=3)
    a = rng.integers(0, 6, size=6)
    b = rng.integers(0, 6, size=6)
    cb = _bounds(1, np.minimum(a, b), np.maximum(a, b) + 1)
    for causal in (False, True):
        O, L = ref(q, k, v, causal=causal, scale=0.9, col_bounds=cb)
        for h in range(2):
            for i in range(5):
                vis = [j for j in range(6) if cb[0, j, 0] <= i < cb[0, j, 1]
                       and (not causal or j <= i + 1)]
                if not vis:
                    assert np.all(O[0, h, i] == 0) and L[0, h, i] == -np.inf
                    continue
                s = [0.9 * sum(q[0, h, i, c] * k[0, 0, j, c] for c in range(3))
                     for j in vis]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for c in range(3):
                    o = sum(wj * v[0, 0, j, c] for wj, j in zip(w, vis)) / z
                    assert abs(O[0, h, i, c] - o) < 1e-12
                assert abs(L[0, h, i] - (m + math.log(z))) < 1e-12


def pin_row_seeing_nothing(ref):
    q, k, v = _qkv(6)
    cb = _bounds(2, np.full(9, 3), np.full(9, 9))   # rows 0..2 see nothing
    O, L = ref(q, k, v, causal=False, scale=0.5, col_bounds=cb)
    assert np.all(O[:, :, :3] == 0) and np.all(np.isneginf(L[:, :, :3]))
    assert np.all(np.isfinite(L[:, :, 3:]))


PINS = [pin_intervals_make_causal, pin_intervals_make_window,
        pin_documents_are_slices, pin_hidden_keys_drop_out, pin_brute_force,
        pin_row_seeing_nothing]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_colmask_pins(pin):
    pin(reference_attention)


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "attention.py")
MUTANTS = {
    "upper_bound_inclusive": ("(rows[:, None] < hi[None, :])",
                              "(rows[:, None] <= hi[None, :])"),
    "bounds_swapped": ("lo, hi = cb[cols, 0], cb[cols, 1]",
                       "hi, lo = cb[cols, 0], cb[cols, 1]"),
    "indexed_by_rows": ("lo, hi = cb[cols, 0], cb[cols, 1]",
                        "lo, hi = cb[np.minimum(cols, rows.max()), 0], cb[np.minimum(cols, rows.max()), 1]"),
    "mask_ignored": ("            if col_bounds is not None:\n",
                     "            if False:\n"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_colmask_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("attention_mutant")
    exec(compile(src.replace(old, new), "attention_mutant", "exec"),
         mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod.reference_attention)
        except Exception:
            failed.append(pin.__name__)
    assert failed, name
