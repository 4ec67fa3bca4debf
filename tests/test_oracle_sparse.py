"""CPU pins of the oracle's block-sparse mask: an all-ones mask is the
dense oracle, a block-diagonal mask is attention on each diagonal block
alone, pure-Python brute force on tiny shapes with random masks, rows
whose blocks are all empty, and planted mistakes these pins must catch."""
import math
import os
import types

import numpy as np
import pytest

from oracle import reference_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

TOL = 1e-12


def _attn(mod=None):
    ref = reference_attention if mod is None else mod.reference_attention

    def f(q, k, v, causal, scale, block_mask, block_size):
        return ref(q, k, v, causal=causal, scale=scale,
                   block_mask=block_mask, block_size=block_size)
    return f


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_all_ones_is_dense(attn):
    rng = np.random.default_rng(70)
    q, k, v = _rand(rng, 2, 4, 9, 3), _rand(rng, 2, 2, 11, 3), _rand(rng, 2, 2, 11, 3)
    for causal in (False, True):
        bm = np.ones((2, 4, 3, 4), np.uint8)
        O, lse = attn(q, k, v, causal, 0.6, bm, (4, 3))
        Od, ld = reference_attention(q, k, v, causal=causal, scale=0.6)
        np.testing.assert_array_equal(O, Od)
        np.testing.assert_array_equal(lse, ld)


def pin_block_diagonal(attn):
    """Blocks of 4 rows x 4 keys on the diagonal only: each group of 4
    queries attends to its own 4 keys, computed on slices."""
    rng = np.random.default_rng(71)
    q, k, v = _rand(rng, 1, 2, 12, 5), _rand(rng, 1, 1, 12, 5), _rand(rng, 1, 1, 12, 5)
    bm = np.eye(3, dtype=np.uint8)[None, None]
    O, lse = attn(q, k, v, False, 0.4, bm, (4, 4))
    for t in range(3):
        sl = slice(4 * t, 4 * t + 4)
        Os, ls = reference_attention(q[:, :, sl], k[:, :, sl], v[:, :, sl],
                                     causal=False, scale=0.4)
        np.testing.assert_allclose(O[:, :, sl], Os, rtol=0, atol=TOL)
        np.testing.assert_allclose(lse[:, :, sl], ls, rtol=0, atol=TOL)


def _brute(q, k, v, causal, scale, bm, bs):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros(q.shape)
    lse = np.full((B, Hq, Nq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk)
                        if bm[b][h][i // bs[0]][j // bs[1]]
                        and (not causal or j <= i + Nk - Nq)]
                if not keys:
                    continue
                s = {j: scale * sum(q[b, h, i, t] * k[b, g, j, t]
                                    for t in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                z = sum(w.values())
                lse[b, h, i] = mx + math.log(z)
                for t in range(d):
                    O[b, h, i, t] = sum(w[j] * v[b, g, j, t] for j in keys) / z
    return O, lse


def pin_brute_force_random_masks(attn):
    rng = np.random.default_rng(72)
    for Nq, Nk, bs in ((5, 7, (2, 3)), (6, 4, (3, 1)), (4, 9, (1, 2))):
        q, k, v = _rand(rng, 1, 2, Nq, 2), _rand(rng, 1, 1, Nk, 2), _rand(rng, 1, 1, Nk, 2)
        nqb, nkb = -(-Nq // bs[0]), -(-Nk // bs[1])
        bm = (rng.random((1, 2, nqb, nkb)) < 0.5).astype(np.uint8)
        for causal in (False, True):
            O, lse = attn(q, k, v, causal, 0.8, bm, bs)
            Ob, lb = _brute(q, k, v, causal, 0.8, bm, bs)
            np.testing.assert_allclose(O, Ob, rtol=0, atol=TOL)
            fin = np.isfinite(lb)
            np.testing.assert_array_equal(np.isfinite(lse), fin)
            np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=TOL)


def pin_empty_block_rows(attn):
    rng = np.random.default_rng(73)
    q, k, v = _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3)
    bm = np.array([[[[1, 1], [0, 0], [1, 0]]]], np.uint8)
    O, lse = attn(q, k, v, False, 0.5, bm, (2, 3))
    assert np.all(O[0, 0, 2:4] == 0) and np.all(np.isneginf(lse[0, 0, 2:4]))
    assert np.all(np.isfinite(lse[0, 0, :2])) and np.all(np.isfinite(lse[0, 0, 4:]))


PINS = [pin_all_ones_is_dense, pin_block_diagonal,
        pin_brute_force_random_masks, pin_empty_block_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_sparse_pins(pin):
    pin(_attn())


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "attention.py")
MUTANTS = {
    "block_sizes_swapped": ("return bm[(rows // bq)[:, None], (cols // bk)[None, :]]",
                            "return bm[(rows // bk)[:, None] % bm.shape[0], (cols // bq)[None, :] % bm.shape[1]]"),
    "mask_transposed": ("return bm[(rows // bq)[:, None], (cols // bk)[None, :]]",
                        "return bm[(cols // bk)[None, :] % bm.shape[0], (rows // bq)[:, None] % bm.shape[1]]"),
    "mask_ignored": ("vis_bh = vis & block_visible(", "vis_bh = vis | block_visible("),
    "mask_inverted": ("bm = np.asarray(block_mask_bh) != 0", "bm = np.asarray(block_mask_bh) == 0"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_sparse_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("sparse_mutant")
    exec(compile(src.replace(old, new), "sparse_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(_attn(mod))
        except Exception:
            failed.append(pin.__name__)
    assert failed, name
