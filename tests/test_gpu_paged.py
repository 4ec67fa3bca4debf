"""Forward over a paged KV cache (fa_fwd_paged) against the float64 paged
oracle: scattered pages, ragged and empty sequences, causal and windowed
masks, several split counts; and, with the pages in order, bit-for-bit
agreement with the contiguous KV-split call."""
import numpy as np
import pytest

from fa_inputs import make_paged
from oracle import paged_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# B, Hq, Hkv, Nq, d, page_size, max_pages, seqlens, causal, window
CASES = [
    (3, 8, 2, 1, 128, 32, 10, [1, 200, 320], False, (-1, -1)),
    (2, 4, 4, 3, 64, 64, 8, [0, 500], True, (-1, -1)),
    (4, 16, 4, 4, 128, 256, 5, [1280, 77, 1000, 256], True, (300, -1)),
    (2, 32, 8, 1, 128, 32, 128, [4096, 2049], False, (-1, -1)),
    (2, 8, 1, 2, 64, 128, 6, [700, 129], False, (100, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}d{c[4]}p{c[5]}x{c[6]}"
                         f"{'-causal' if c[8] else ''}-w{c[9][0]},{c[9][1]}")
def test_paged_matches_oracle(case):
    B, Hq, Hkv, Nq, d, P, maxp, lens, causal, window = case
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, d, P, maxp, lens, seed=41)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    args = (dev(q), dev(kc), dev(vc), _i32(table), _i32(sl))
    ops = _ops()
    o32, l32 = ops.fa_fwd_paged(*args, causal=causal, scale=scale,
                                window=window, out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd_paged(*args, causal=causal, scale=scale,
                                window=window, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = paged_attention(f64(q), f64(kc), f64(vc), table, sl,
                                   causal=causal, scale=scale, window=window)
    compare(host(o32), host(l32), O_ref, L_ref, what=f"paged {case}")


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_paged_split_counts(splits):
    B, Hq, Hkv, Nq, d, P, maxp = 2, 8, 2, 2, 128, 64, 12
    lens = [768, 300]
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, d, P, maxp, lens, seed=42)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_paged(dev(q), dev(kc), dev(vc), _i32(table),
                                 _i32(sl), causal=True, scale=scale,
                                 out_dtype=torch.float32, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = paged_attention(f64(q), f64(kc), f64(vc), table, sl,
                                   causal=True, scale=scale)
    compare(host(o), host(lse), O_ref, L_ref, what=f"{splits} splits")


def test_in_order_pages_match_contiguous_splitkv():
    """One sequence per batch entry whose pages are 0, 1, 2, ... of its own
    slice of the pool holds the rows of a contiguous cache; with the same
    split count the paged call reproduces fa_fwd_splitkv bit for bit."""
    B, Hq, Hkv, Nq, d, P, maxp = 2, 8, 2, 1, 128, 64, 16
    N = P * maxp
    rng = np.random.default_rng(43)
    from fa_inputs import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32))
    # pool page b * maxp + j holds rows j P .. j P + P - 1 of batch entry b
    kc = k.transpose(0, 2, 1, 3).reshape(B * maxp, P, Hkv, d)
    vc = v.transpose(0, 2, 1, 3).reshape(B * maxp, P, Hkv, d)
    table = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp)
    sl = np.full(B, N, dtype=np.int32)
    ops = _ops()
    splits = ops.paged_num_splits(B, Hq, Hkv, Nq, d, P, maxp)
    o1, l1 = ops.fa_fwd_paged(dev(q), dev(kc), dev(vc), _i32(table), _i32(sl),
                              out_dtype=torch.float32, num_splits=splits)
    o2, l2 = ops.fa_fwd_splitkv(dev(q), dev(k), dev(v), splits,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
