"""Variable-length decode over a padded contiguous cache (fa_fwd_kvlen)
against the float64 oracle: ragged, empty and full lengths, GQA, several
queries per sequence, causal and windowed masks, several split counts; the
padding rows hold NaN so that reading one shows; and at full lengths,
bit-for-bit agreement with the KV-split call without lengths."""
import numpy as np
import pytest

from fa_inputs import make_qkv
from oracle import kvlen_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAN_BF16 = np.uint16(0x7FC0)


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _case(B, Hq, Hkv, Nq, Nk, d, lens, seed):
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=seed)
    k, v = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k[b, :, n:] = NAN_BF16
        v[b, :, n:] = NAN_BF16
    return q, k, v


# B, Hq, Hkv, Nq, Nk (padded), d, lengths, causal, window
CASES = [
    (3, 8, 2, 1, 320, 128, [1, 200, 320], False, (-1, -1)),
    (2, 4, 4, 3, 512, 64, [0, 500], True, (-1, -1)),
    (4, 16, 4, 4, 1280, 128, [1280, 77, 1000, 256], True, (300, -1)),
    (2, 32, 8, 1, 4096, 128, [4096, 2049], False, (-1, -1)),
    (2, 8, 1, 2, 700, 64, [700, 129], False, (100, 0)),
    (5, 8, 8, 1, 96, 128, [33, 0, 96, 31, 64], True, (-1, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}k{c[4]}d{c[5]}"
                         f"{'-causal' if c[7] else ''}-w{c[8][0]},{c[8][1]}")
def test_kvlen_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, lens, causal, window = case
    print(f"kvlen case {case}", flush=True)
    q, k, v = _case(B, Hq, Hkv, Nq, Nk, d, lens, seed=51)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    args = (dev(q), dev(k), dev(v), _i32(lens))
    ops = _ops()
    o32, l32 = ops.fa_fwd_kvlen(*args, causal=causal, scale=scale,
                                window=window, out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd_kvlen(*args, causal=causal, scale=scale,
                                window=window, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = kvlen_attention(f64(q), f64(k), f64(v), lens,
                                   causal=causal, scale=scale, window=window)
    compare(host(o32), host(l32), O_ref, L_ref, what=f"kvlen {case}")


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_kvlen_split_counts(splits):
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 2, 768, 128
    lens = [768, 300]
    q, k, v = _case(B, Hq, Hkv, Nq, Nk, d, lens, seed=52)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_kvlen(dev(q), dev(k), dev(v), _i32(lens),
                                 causal=True, scale=scale,
                                 out_dtype=torch.float32, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = kvlen_attention(f64(q), f64(k), f64(v), lens, causal=True,
                                   scale=scale)
    compare(host(o), host(lse), O_ref, L_ref, what=f"{splits} splits")


def test_full_lengths_match_splitkv():
    """Every sequence at the padded length: the KV-split call without
    lengths, bit for bit, at the same split count."""
    B, Hq, Hkv, Nq, Nk, d = 3, 8, 2, 1, 1000, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=53)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ops = _ops()
    o1, l1 = ops.fa_fwd_kvlen(dev(q), dev(k), dev(v), _i32([Nk] * B),
                              causal=True, scale=scale, num_splits=5)
    o2, l2 = ops.fa_fwd_splitkv(dev(q), dev(k), dev(v), 5, causal=True,
                                scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lengths_are_clamped():
    """Lengths past the padded size read as the padded size, negative ones
    as zero (no access outside the cache)."""
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 1, 128, 64
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=54)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_kvlen(dev(q), dev(k), dev(v), _i32([1 << 20, -5]),
                                 causal=False, scale=scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = kvlen_attention(f64(q), f64(k), f64(v), [Nk, 0],
                                   causal=False, scale=scale)
    compare(host(o), host(lse), O_ref, L_ref, what="clamped lengths")
