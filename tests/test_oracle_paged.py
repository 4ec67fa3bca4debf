"""CPU pins of the paged-cache oracle: an in-order page table over a
contiguous cache is the contiguous layout, moving pages around (with the
table) changes nothing, explicit row-by-row lookups, and planted mistakes
that these pins must catch."""
import os
import types

import numpy as np
import pytest

from oracle import paged_attention, paged_rows, reference_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed, B=3, Hq=4, Hkv=2, Nq=2, d=5, P=4, pages_per_seq=5):
    rng = np.random.default_rng(seed)
    num_pages = B * pages_per_seq + 3
    kc = rng.standard_normal((num_pages, P, Hkv, d))
    vc = rng.standard_normal((num_pages, P, Hkv, d))
    q = rng.standard_normal((B, Hq, Nq, d))
    table = rng.permutation(num_pages)[:B * pages_per_seq].reshape(
        B, pages_per_seq)
    seqlen = rng.integers(1, P * pages_per_seq + 1, size=B)
    return q, kc, vc, table, seqlen


def _paged(mod=None):
    f = paged_attention if mod is None else mod.paged_attention
    return f


def pin_in_order_table_is_contiguous(attn):
    """Pages 0, 1, 2, ... of a cache that holds one sequence's rows in order
    give exactly the contiguous forward oracle on those rows."""
    rng = np.random.default_rng(1)
    P, n_pages, Hkv, d, n = 4, 6, 2, 3, 21
    k = rng.standard_normal((1, Hkv, n_pages * P, d))
    v = rng.standard_normal((1, Hkv, n_pages * P, d))
    q = rng.standard_normal((1, 4, 3, d))
    kc = k[0].transpose(1, 0, 2).reshape(n_pages, P, Hkv, d)
    vc = v[0].transpose(1, 0, 2).reshape(n_pages, P, Hkv, d)
    for causal in (False, True):
        O, lse = attn(q, kc, vc, np.arange(n_pages)[None], np.array([n]),
                      causal=causal, scale=0.6)
        Oc, lc = reference_attention(q, k[:, :, :n], v[:, :, :n],
                                     causal=causal, scale=0.6)
        np.testing.assert_array_equal(O, Oc)
        np.testing.assert_array_equal(lse, lc)


def pin_moving_pages_changes_nothing(attn):
    """Permuting the physical pages and the table with them leaves the
    result unchanged; so does garbage in pages no sequence owns."""
    q, kc, vc, table, seqlen = _case(2)
    O, lse = attn(q, kc, vc, table, seqlen, causal=True, scale=0.5)
    perm = np.random.default_rng(3).permutation(kc.shape[0])
    inv = np.argsort(perm)
    kc2, vc2 = kc[perm].copy(), vc[perm].copy()    # new page p = old perm[p]
    table2 = inv[table]
    used = set(table2.ravel().tolist())
    for p in range(kc2.shape[0]):
        if p not in used:
            kc2[p] = 1e3
            vc2[p] = -1e3
    O2, lse2 = attn(q, kc2, vc2, table2, seqlen, causal=True, scale=0.5)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def pin_row_lookup_by_hand(attn):
    """Each sequence against the contiguous oracle on rows gathered with an
    explicit loop over (page, slot)."""
    q, kc, vc, table, seqlen = _case(4)
    P = kc.shape[1]
    O, lse = attn(q, kc, vc, table, seqlen, causal=False, scale=0.7)
    for b in range(q.shape[0]):
        n = int(seqlen[b])
        k = np.stack([kc[table[b][r // P], r % P] for r in range(n)])
        v = np.stack([vc[table[b][r // P], r % P] for r in range(n)])
        Ob, lb = reference_attention(q[b:b + 1], k.transpose(1, 0, 2)[None],
                                     v.transpose(1, 0, 2)[None], causal=False,
                                     scale=0.7)
        np.testing.assert_array_equal(O[b], Ob[0])
        np.testing.assert_array_equal(lse[b], lb[0])


def pin_empty_sequence(attn):
    q, kc, vc, table, seqlen = _case(5)
    seqlen = seqlen.copy()
    seqlen[1] = 0
    O, lse = attn(q, kc, vc, table, seqlen, causal=True, scale=0.5)
    assert np.all(O[1] == 0) and np.all(np.isneginf(lse[1]))


PINS = [pin_in_order_table_is_contiguous, pin_moving_pages_changes_nothing,
        pin_row_lookup_by_hand, pin_empty_sequence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_paged_pins(pin):
    pin(_paged())


def test_paged_rows_rejects_bad_pages():
    kc = np.zeros((3, 4, 1, 2))
    with pytest.raises(ValueError):
        paged_rows(kc, np.array([0, 5]), 6)


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "paged.py")
MUTANTS = {
    "slot_from_page_count": ("rows[r] = cache[page, r % page_size]",
                             "rows[r] = cache[page, r % num_pages]"),
    "page_index_off_by_one": ("page = int(page_table_row[r // page_size])",
                              "page = int(page_table_row[r // page_size + 1]) if r // page_size + 1 < len(page_table_row) else 0"),
    "table_ignored": ("page = int(page_table_row[r // page_size])",
                      "page = r // page_size"),
    "seqlen_ignored": ("n = int(seqlen_k[b])", "n = len(page_table[b]) * k_cache.shape[1]"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_paged_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("paged_mutant")
    exec(compile(src.replace(old, new), "paged_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(_paged(mod))
        except Exception:
            failed.append(pin.__name__)
    assert failed, name
