"""Forward with a column-interval mask (fa_fwd_colmask) against the float64
oracle: document masks (causal and bidirectional inside documents), a
prefix-LM mask, random intervals (some empty), bounds outside [0, Nq) and
reversed intervals, Nq != Nk and ragged sizes, GQA, d = 32 to 128, a zero
scale; sampled rows of a long packed-document sequence; and, with every key
visible to every row, bit-for-bit agreement with fa_fwd."""
import numpy as np
import pytest

from fa_inputs import (document_column_bounds, make_qkv,
                       prefix_lm_column_bounds, random_column_bounds,
                       random_doc_lens)
from oracle import reference_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _bounds(kind, B, Nq, Nk, seed):
    out = []
    for b in range(B):
        if kind == "docs_causal":
            out.append(document_column_bounds(random_doc_lens(Nk, 40, 400, seed=seed + b)))
        elif kind == "docs_bidir":
            out.append(document_column_bounds(random_doc_lens(Nk, 40, 400, seed=seed + b),
                                              causal_docs=False))
        elif kind == "prefix":
            out.append(prefix_lm_column_bounds(Nk, 100 + 37 * b))
        elif kind == "wild":
            # bounds outside [0, Nq) and reversed (empty) intervals
            rng = np.random.default_rng(seed + b)
            out.append(rng.integers(-300, Nq + 300, size=(Nk, 2)))
        else:
            out.append(random_column_bounds(Nq, Nk, seed=seed + b))
    return np.ascontiguousarray(np.stack(out), dtype=np.int32)


# B, Hq, Hkv, Nq, Nk, d, causal, kind
CASES = [
    (1, 8, 2, 1000, 1000, 128, True, "docs_causal"),
    (2, 4, 4, 777, 777, 64, False, "docs_bidir"),
    (1, 4, 2, 600, 600, 128, False, "prefix"),
    (2, 4, 1, 300, 520, 128, False, "random"),
    (1, 8, 8, 500, 777, 64, True, "random"),
    (1, 4, 2, 257, 257, 128, True, "docs_bidir"),
    (1, 4, 2, 600, 600, 96, True, "docs_causal"),
    (1, 4, 4, 500, 777, 32, False, "random"),
    (1, 4, 2, 300, 900, 128, True, "random"),
    (1, 4, 2, 513, 513, 64, True, "wild"),
    (1, 4, 2, 700, 700, 128, False, "wild"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}k{c[4]}d{c[5]}"
                         f"{'-causal' if c[6] else ''}-{c[7]}")
def test_colmask_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, causal, kind = case
    print(f"colmask case {case}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=61)
    cb = _bounds(kind, B, Nq, Nk, seed=62)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ops = _ops()
    CB = torch.from_numpy(cb).cuda()
    o32, l32 = ops.fa_fwd_colmask(dev(q), dev(k), dev(v), CB, causal=causal,
                                  scale=scale, out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd_colmask(dev(q), dev(k), dev(v), CB, causal=causal,
                                  scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale, col_bounds=cb)
    compare(host(o32), host(l32), O_ref, L_ref, what=f"colmask {case}")


def test_colmask_long_documents_sampled_rows():
    """32 heads over 8 KV heads, 8192 packed tokens in causal documents of
    300 .. 2500 tokens: sampled rows against the oracle."""
    B, Hq, Hkv, N, d = 1, 32, 8, 8192, 128
    print("colmask long documents", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=63)
    cb = np.ascontiguousarray(
        document_column_bounds(random_doc_lens(N, 300, 2500, seed=64))[None])
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_colmask(dev(q), dev(k), dev(v),
                                   torch.from_numpy(cb).cuda(), causal=True,
                                   scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([
        np.random.default_rng(65).choice(N, 40, replace=False),
        [0, 1, 255, 256, N - 1]]))
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=True,
                                       scale=scale, rows=rows, col_bounds=cb)
    compare(host(o)[:, :, rows], host(lse)[:, :, rows], O_ref, L_ref,
            what="long documents")


@pytest.mark.parametrize("causal", [False, True])
def test_all_visible_matches_fa_fwd(causal):
    B, Hq, Hkv, N, d = 2, 8, 2, 700, 128
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=66)
    cb = np.zeros((B, N, 2), dtype=np.int32)
    cb[:, :, 1] = N
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ops = _ops()
    o1, l1 = ops.fa_fwd_colmask(dev(q), dev(k), dev(v),
                                torch.from_numpy(cb).cuda(), causal=causal,
                                scale=scale)
    o2, l2 = ops.fa_fwd(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_colmask_zero_scale():
    """Scale 0: every visible key has the same weight, so each row is the
    mean of the V rows it sees (hidden keys must still get weight 0)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 900, 128
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=67)
    cb = _bounds("docs_causal", B, N, N, seed=68)
    o, lse = _ops().fa_fwd_colmask(dev(q), dev(k), dev(v),
                                   torch.from_numpy(cb).cuda(), causal=True,
                                   scale=0.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=True,
                                       scale=0.0, col_bounds=cb)
    compare(host(o), host(lse), O_ref, L_ref, what="colmask scale 0")
