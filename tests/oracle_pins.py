"""Checks that pin an attention-forward implementation to facts fixed by the
mathematics and by the pages, independent of that implementation.

Each ``pin_*`` takes ``attn(q, k, v, causal, scale) -> (O, lse)`` working on
float64 arrays shaped [B, H, N, d] and raises AssertionError on a mismatch.
The test suite runs them against the oracle's three forms (definition,
tiled online softmax, KV split + merge) and against deliberately broken
copies of the oracle, which must each fail at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------ hand examples
def pin_hand_two_keys(attn):
    """One query, two keys, d = 1, scale 1: scores 0 and ln 3 give weights
    1/4 and 3/4; values 4 and 8 give O = 7; lse = ln(1 + 3) = ln 4."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.0], [math.log(3.0)]]]])
    v = np.array([[[[4.0], [8.0]]]])
    O, lse = attn(q, k, v, False, 1.0)
    _close(O, [[[[7.0]]]], 1e-13, "O")
    _close(lse, [[[math.log(4.0)]]], 1e-13, "lse")


def pin_hand_scale_and_causal(attn):
    """Two queries, two keys, d = 2, scale 1/2, causal.

    q0 = (2, 0), q1 = (0, 2); k0 = (0, 0), k1 = (0, 2 ln 2) -> scaled scores
    row 0: (0, 0) but key 1 hidden -> weight (1, 0), O0 = v0, lse0 = 0;
    row 1: (0, 2 ln 2) -> exp = (1, 4), weights (1/5, 4/5), lse1 = ln 5.
    v0 = (10, -5), v1 = (0, 5) -> O1 = (2, 3).
    """
    q = np.array([[[[2.0, 0.0], [0.0, 2.0]]]])
    k = np.array([[[[0.0, 0.0], [0.0, 2.0 * math.log(2.0)]]]])
    v = np.array([[[[10.0, -5.0], [0.0, 5.0]]]])
    O, lse = attn(q, k, v, True, 0.5)
    _close(O, [[[[10.0, -5.0], [2.0, 3.0]]]], 1e-13, "O")
    _close(lse, [[[0.0, math.log(5.0)]]], 1e-13, "lse")
    # non-causal row 0 now sees both keys at equal score 0: O0 = (5, 0)
    O, lse = attn(q, k, v, False, 0.5)
    _close(O[0, 0, 0], [5.0, 0.0], 1e-13, "O row0 non-causal")
    _close(lse[0, 0, 0], math.log(2.0), 1e-13, "lse row0 non-causal")


def pin_hand_gqa(attn):
    """Two query heads over one KV head: both read the same keys/values.
    Head 0 query picks key 0 strongly, head 1 query picks key 1."""
    big = 60.0
    q = np.array([[[[big, 0.0]], [[0.0, big]]]])          # [1, 2, 1, 2]
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])            # [1, 1, 2, 2]
    v = np.array([[[[3.0, 1.0], [-2.0, 7.0]]]])
    O, lse = attn(q, k, v, False, 1.0)
    e = math.exp(-big)
    w = 1.0 / (1.0 + e)
    _close(O[0, 0, 0], [3.0 * w - 2.0 * (1 - w), 1.0 * w + 7.0 * (1 - w)],
           1e-12, "head0")
    _close(O[0, 1, 0], [3.0 * (1 - w) - 2.0 * w, 1.0 * (1 - w) + 7.0 * w],
           1e-12, "head1")
    _close(lse[0, :, 0], [big + math.log1p(e)] * 2, 1e-12, "lse")


def pin_hand_bottom_right_causal(attn):
    """Nq = 2 queries against Nk = 4 keys with the causal flag: query 0 sees
    keys 0..2, query 1 sees keys 0..3 (alignment at the last key).  With
    scale 0 every visible key weighs the same."""
    q = np.ones((1, 1, 2, 1))
    k = np.zeros((1, 1, 4, 1))
    v = np.arange(4.0).reshape(1, 1, 4, 1)
    O, lse = attn(q, k, v, True, 0.0)
    _close(O[0, 0, :, 0], [1.0, 1.5], 1e-13, "O")
    _close(lse[0, 0], [math.log(3.0), math.log(4.0)], 1e-13, "lse")


def pin_brute_force_loops(attn, seed=0):
    """Pure-Python loops over tiny shapes (Nq, Nk <= 3, d <= 3, GQA 2:1),
    exponentials and sums taken one at a time."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 3, 3, 3
        q, k, v = _rand(rng, B, Hq, Nq, d), _rand(rng, B, Hkv, Nk, d), \
            _rand(rng, B, Hkv, Nk, d)
        scale = 0.7
        O, lse = attn(q, k, v, causal, scale)
        for h in range(Hq):
            for i in range(Nq):
                scores = []
                for j in range(Nk):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += q[0, h, i, c] * k[0, 0, j, c]
                    scores.append((j, scale * dot))
                top = max(s for _, s in scores)
                tot = 0.0
                for _, s in scores:
                    tot += math.exp(s - top)
                out = [0.0] * d
                for j, s in scores:
                    wgt = math.exp(s - top) / tot
                    for c in range(d):
                        out[c] += wgt * v[0, 0, j, c]
                _close(O[0, h, i], out, 1e-12, f"O h{h} i{i}")
                _close(lse[0, h, i], top + math.log(tot), 1e-12, f"lse h{h} i{i}")


# ------------------------------------------------------------ closed forms
def _visible_counts(Nq, Nk, causal):
    i = np.arange(Nq)
    return np.full(Nq, Nk) if not causal else np.clip(i + (Nk - Nq) + 1, 0, Nk)


def _mean_visible_v(v_head, Nq, Nk, causal):
    cs = np.cumsum(v_head, axis=0)
    n = _visible_counts(Nq, Nk, causal)
    out = np.zeros((Nq, v_head.shape[1]))
    for i in range(Nq):
        if n[i] > 0:
            out[i] = cs[n[i] - 1] / n[i]
    return out


def pin_scale_zero(attn, seed=1):
    """scale = 0: every visible key has weight 1/#visible, so O_i is the
    mean of the visible V rows and lse_i = ln #visible."""
    rng = np.random.default_rng(seed)
    for causal, (Nq, Nk) in ((False, (5, 7)), (True, (6, 6)), (True, (3, 8))):
        q, k, v = _rand(rng, 2, 4, Nq, 3), _rand(rng, 2, 2, Nk, 3), \
            _rand(rng, 2, 2, Nk, 3)
        O, lse = attn(q, k, v, causal, 0.0)
        for b in range(2):
            for h in range(4):
                _close(O[b, h], _mean_visible_v(v[b, h // 2], Nq, Nk, causal),
                       1e-12, "O")
                _close(lse[b, h], np.log(_visible_counts(Nq, Nk, causal)),
                       1e-12, "lse")


def pin_identical_keys(attn, seed=2):
    """All keys equal to one vector u: all visible scores of row i equal
    s_i = scale * q_i . u, so O_i = mean of visible V rows and
    lse_i = s_i + ln #visible."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        Nq = Nk = 9
        d = 4
        q = _rand(rng, 1, 2, Nq, d)
        u = rng.standard_normal(d)
        k = np.broadcast_to(u, (1, 1, Nk, d)).copy()
        v = _rand(rng, 1, 1, Nk, d)
        scale = 0.9
        O, lse = attn(q, k, v, causal, scale)
        for h in range(2):
            _close(O[0, h], _mean_visible_v(v[0, 0], Nq, Nk, causal), 1e-12, "O")
            s = scale * (q[0, h] @ u)
            _close(lse[0, h], s + np.log(_visible_counts(Nq, Nk, causal)),
                   1e-12, "lse")


def pin_one_hot(attn, seed=3):
    """q_i = c e_a and key j* = c e_a, every other key orthogonal to e_a:
    the score gap c^2 * scale >= 40 makes O_i = v_{j*} to ~N e^-40."""
    rng = np.random.default_rng(seed)
    d, Nk = 8, 6
    c = 18.0
    scale = 1.0 / 8.0                     # c^2 * scale = 40.5
    for jstar in range(Nk):
        a = jstar % d
        q = np.zeros((1, 1, 1, d))
        q[0, 0, 0, a] = c
        k = _rand(rng, 1, 1, Nk, d)
        k[..., a] = 0.0
        k[0, 0, jstar] = 0.0
        k[0, 0, jstar, a] = c
        v = _rand(rng, 1, 1, Nk, d)
        O, lse = attn(q, k, v, False, scale)
        _close(O[0, 0, 0], v[0, 0, jstar], Nk * math.exp(-40.0) * 10, "O")
        _close(lse[0, 0, 0], c * c * scale, Nk * math.exp(-40.0), "lse")


def pin_convex_hull(attn, seed=4):
    """Each O row is a convex combination of the visible V rows, so each
    coordinate lies between their minimum and maximum."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        Nq, Nk, d = 7, 7, 5
        q, k, v = 3 * _rand(rng, 1, 2, Nq, d), 3 * _rand(rng, 1, 2, Nk, d), \
            _rand(rng, 1, 2, Nk, d)
        O, _ = attn(q, k, v, causal, 1.0)
        n = _visible_counts(Nq, Nk, causal)
        for h in range(2):
            for i in range(Nq):
                vv = v[0, h, : n[i]]
                assert np.all(O[0, h, i] >= vv.min(axis=0) - 1e-12)
                assert np.all(O[0, h, i] <= vv.max(axis=0) + 1e-12)


def pin_shift_invariance(attn, seed=5):
    """Replacing K by K + 1 u^T adds kappa_i = scale * q_i . u to every
    score of row i: O is unchanged and lse_i grows by kappa_i."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        Nq, Nk, d = 6, 6, 4
        q, k, v = _rand(rng, 1, 2, Nq, d), _rand(rng, 1, 1, Nk, d), \
            _rand(rng, 1, 1, Nk, d)
        u = rng.standard_normal(d) * 5
        scale = 0.8
        O0, lse0 = attn(q, k, v, causal, scale)
        O1, lse1 = attn(q, k + u, v, causal, scale)
        _close(O1, O0, 1e-11, "O")
        kappa = scale * np.einsum("bhid,d->bhi", q, u)
        _close(lse1, lse0 + kappa, 1e-11, "lse")


def pin_gqa_equals_replicated(attn, seed=6):
    """Grouped KV heads give exactly what the same heads replicated
    contiguously (each KV head repeated Hq/Hkv times) give as full MHA."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 6, 2, 5, 3
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), \
        _rand(rng, B, Hkv, N, d)
    for causal in (False, True):
        Og, lg = attn(q, k, v, causal, 0.6)
        rep = Hq // Hkv
        Om, lm = attn(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1),
                      causal, 0.6)
        _close(Og, Om, 1e-13, "O")
        _close(lg, lm, 1e-13, "lse")
        # and head hq of the group really reads KV head hq // rep
        for h in range(Hq):
            Oh, _ = attn(q[:, h:h + 1], k[:, h // rep:h // rep + 1],
                         v[:, h // rep:h // rep + 1], causal, 0.6)
            _close(Og[:, h:h + 1], Oh, 1e-13, "per-head")


def pin_key_permutation(attn, seed=7):
    """Without a mask the result does not depend on the order of the keys,
    as long as K and V rows are permuted together."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 2, 9, 3), \
        _rand(rng, 1, 2, 9, 3)
    perm = rng.permutation(9)
    O0, l0 = attn(q, k, v, False, 1.1)
    O1, l1 = attn(q, k[:, :, perm], v[:, :, perm], False, 1.1)
    _close(O1, O0, 1e-12, "O")
    _close(l1, l0, 1e-12, "lse")
    # the value rows must follow their keys: permuting V alone changes O
    O2, _ = attn(q, k, v[:, :, perm], False, 1.1)
    assert np.max(np.abs(O2 - O0)) > 1e-3


def pin_causal_first_row(attn, seed=8):
    """Under the causal mask (Nq = Nk) query 0 sees key 0 only: O_0 = v_0
    and lse_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 5, 4), \
        _rand(rng, 1, 1, 5, 4)
    O, lse = attn(q, k, v, True, 0.3)
    _close(O[0, 0, 0], v[0, 0, 0], 1e-13, "O0")
    _close(lse[0, 0, 0], 0.3 * (q[0, 0, 0] @ k[0, 0, 0]), 1e-13, "lse0")


def pin_large_scores(attn):
    """Scores near +-1000 do not overflow: the row max is subtracted before
    exponentiation, so the result is the finite limit."""
    q = np.array([[[[1000.0], [-1000.0]]]])
    k = np.array([[[[1.0], [0.999], [-1.0]]]])
    v = np.array([[[[1.0], [2.0], [3.0]]]])
    O, lse = attn(q, k, v, False, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    # row 0: gap 1 between the first two keys -> weights 1/(1+e^-1), ...
    w = 1.0 / (1.0 + math.exp(-1.0) + math.exp(-2000.0))
    _close(O[0, 0, 0, 0], w * (1.0 + 2.0 * math.exp(-1.0)), 1e-12, "O row0")
    _close(lse[0, 0, 0], 1000.0 + math.log1p(math.exp(-1.0)), 1e-9, "lse row0")
    _close(O[0, 0, 1, 0], 3.0, 1e-12, "O row1")


def pin_fully_masked_rows(attn):
    """Causal with Nq > Nk: the first Nq - Nk queries see no key at all; by
    the documented reading their O is 0 and lse is -inf."""
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 1, 1, 5, 2), _rand(rng, 1, 1, 3, 2), \
        _rand(rng, 1, 1, 3, 2)
    O, lse = attn(q, k, v, True, 1.0)
    assert np.all(O[0, 0, :2] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    _close(O[0, 0, 2], v[0, 0, 0], 1e-13, "first row with a key")


ALL_PINS = [
    pin_hand_two_keys, pin_hand_scale_and_causal, pin_hand_gqa,
    pin_hand_bottom_right_causal, pin_brute_force_loops, pin_scale_zero,
    pin_identical_keys, pin_one_hot, pin_convex_hull, pin_shift_invariance,
    pin_gqa_equals_replicated, pin_key_permutation, pin_causal_first_row,
    pin_large_scores, pin_fully_masked_rows,
]
