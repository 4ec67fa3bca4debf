"""CPU pins of the padded-cache oracle (sequences of unequal cache length in
one [B, Hkv, Nk_max, d] tensor): full lengths are the plain forward oracle
on the whole batch, padding rows are never read, the causal alignment sits
at each sequence's own last key (checked against the plain oracle on a cut
cache), an empty sequence, and planted mistakes that these pins catch."""
import os
import types

import numpy as np
import pytest

from oracle import kvlen_attention, reference_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed, B=3, Hq=4, Hkv=2, Nq=3, Nk=11, d=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    return q, k, v


def pin_full_lengths_are_the_batch(attn):
    """Every sequence at the full cache length: the plain oracle."""
    q, k, v = _case(1)
    for causal in (False, True):
        O, L = attn(q, k, v, np.full(3, 11), causal=causal, scale=0.4)
        Or, Lr = reference_attention(q, k, v, causal=causal, scale=0.4)
        np.testing.assert_allclose(O, Or, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-12)


def pin_padding_is_never_read(attn):
    """Rows past a sequence's length may hold anything."""
    q, k, v = _case(2)
    lens = np.array([4, 11, 7])
    O, L = attn(q, k, v, lens, causal=True, scale=0.3)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k2[b, :, n:] = 1e3 * np.sign(k2[b, :, n:])
        v2[b, :, n:] = -7.0
    O2, L2 = attn(q, k2, v2, lens, causal=True, scale=0.3)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)


def pin_alignment_at_own_last_key(attn):
    """Causal, Nq queries, length n: query i sees keys 0 .. n - Nq + i,
    which is the non-causal oracle on a cache cut to n - Nq + i + 1 rows,
    and each sequence equals the plain oracle on its own cut cache."""
    q, k, v = _case(3, B=2, Nq=2, Nk=9)
    lens = np.array([5, 9])
    O, L = attn(q, k, v, lens, causal=True, scale=0.5)
    for b, n in enumerate(lens):
        for i in range(2):
            m = n - 2 + i + 1
            Oi, Li = reference_attention(q[b:b + 1, :, i:i + 1],
                                         k[b:b + 1, :, :m], v[b:b + 1, :, :m],
                                         causal=False, scale=0.5)
            np.testing.assert_allclose(O[b, :, i], Oi[0, :, 0], atol=1e-12)
            np.testing.assert_allclose(L[b, :, i], Li[0, :, 0], atol=1e-12)


def pin_window_at_own_last_key(attn):
    """A window of 2 keys to the left: query i of a length-n sequence sees
    keys n - Nq + i - 2 .. n - Nq + i."""
    q, k, v = _case(4, B=2, Nq=2, Nk=10)
    lens = np.array([6, 10])
    O, _ = attn(q, k, v, lens, causal=True, scale=0.5, window=(2, 0))
    for b, n in enumerate(lens):
        for i in range(2):
            c = n - 2 + i
            Oi, _ = reference_attention(q[b:b + 1, :, i:i + 1],
                                        k[b:b + 1, :, c - 2:c + 1],
                                        v[b:b + 1, :, c - 2:c + 1],
                                        causal=False, scale=0.5)
            np.testing.assert_allclose(O[b, :, i], Oi[0, :, 0], atol=1e-12)


def pin_empty_sequence(attn):
    q, k, v = _case(5)
    O, L = attn(q, k, v, np.array([0, 3, 11]), causal=False, scale=0.2)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(L[1:]))


PINS = [pin_full_lengths_are_the_batch, pin_padding_is_never_read,
        pin_alignment_at_own_last_key, pin_window_at_own_last_key,
        pin_empty_sequence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_kvlen_pins(pin):
    pin(kvlen_attention)


def test_kvlen_rejects_bad_length():
    q, k, v = _case(6)
    with pytest.raises(ValueError):
        kvlen_attention(q, k, v, np.array([1, 12, 3]), causal=False, scale=1.0)


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "paged.py")
MUTANTS = {
    "length_ignored": ("length = int(seqlen_k[b])",
                       "length = int(k.shape[2])"),
    "padding_read": ("k[b:b + 1, :, :length],\n",
                     "k[b:b + 1, :, :length] if length == k.shape[2] else k[b:b + 1, :, 1:length + 1],\n"),
    "values_uncut": ("v[b:b + 1, :, :length], causal=causal,",
                     "v[b:b + 1, :, k.shape[2] - length:], causal=causal,"),
    "empty_not_skipped": ("        if length == 0:\n            continue\n        Ob, lb",
                          "        Ob, lb"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_kvlen_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("kvlen_mutant")
    exec(compile(src.replace(old, new), "kvlen_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod.kvlen_attention)
        except Exception:
            failed.append(pin.__name__)
    assert failed, name
