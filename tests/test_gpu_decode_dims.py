"""Head dimensions 32 and 256 in the KV-split (decode) form against the
float64 oracles: the contiguous call (several split counts, causal, several
queries per sequence, GQA, several 32-row tiles of packed rows), a paged
cache and a padded cache of unequal lengths (NaN padding), and a sliding
window; bf16 outputs are the round-to-nearest-even of the fp32 ones."""
import numpy as np
import pytest

from fa_inputs import make_paged, make_qkv
from oracle import kvlen_attention, paged_attention, reference_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DIMS = [32, 256]


def _scale(D):
    return float(np.float32(1.0 / np.sqrt(D)))


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# B, Hq, Hkv, Nq, Nk, causal, splits
CASES = [(2, 8, 2, 1, 1000, False, 4), (1, 4, 4, 3, 777, True, 1),
         (2, 16, 4, 4, 2048, True, 7), (3, 8, 8, 1, 65, False, 2),
         # several 32-row tiles of packed (query, head) rows per KV head
         (1, 16, 2, 9, 1500, True, 3), (2, 32, 4, 5, 2000, True, 5)]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}k{c[4]}"
                         f"{'-causal' if c[5] else ''}-s{c[6]}")
def test_splitkv_dims_match_oracle(case, D):
    B, Hq, Hkv, Nq, Nk, causal, splits = case
    SCALE = _scale(D)
    print(f"d{D} splitkv {case}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, D, seed=71)
    ops = _ops()
    o32, l32 = ops.fa_fwd_splitkv(dev(q), dev(k), dev(v), splits,
                                  causal=causal, scale=SCALE,
                                  out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd_splitkv(dev(q), dev(k), dev(v), splits,
                                  causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(l32, l16)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=SCALE)
    compare(host(o32), host(l32), O_ref, L_ref, what=f"d{D} {case}")


@pytest.mark.parametrize("D", DIMS)
def test_paged_dims_match_oracle(D):
    """fp32 output against the oracle; the bf16 output of the same call is
    the round-to-nearest-even of the fp32 one, with the same lse."""
    SCALE = _scale(D)
    B, Hq, Hkv, Nq, P, maxp = 3, 8, 2, 2, 64, 10
    lens = [1, 400, 640]
    print(f"d{D} paged", flush=True)
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, D, P, maxp, lens,
                                      seed=72)
    args = (dev(q), dev(kc), dev(vc), _i32(table), _i32(sl))
    o, lse = _ops().fa_fwd_paged(*args, causal=True, scale=SCALE,
                                 out_dtype=torch.float32)
    o16, l16 = _ops().fa_fwd_paged(*args, causal=True, scale=SCALE,
                                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(lse, l16)
    O_ref, L_ref = paged_attention(f64(q), f64(kc), f64(vc), table, sl,
                                   causal=True, scale=SCALE)
    compare(host(o), host(lse), O_ref, L_ref, what=f"d{D} paged")


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("window", [(-1, -1), (200, 0)])
def test_kvlen_dims_match_oracle(window, D):
    SCALE = _scale(D)
    B, Hq, Hkv, Nq, Nk = 3, 8, 2, 2, 900
    lens = [900, 0, 333]
    print(f"d{D} kvlen {window}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, D, seed=73)
    k, v = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k[b, :, n:] = np.uint16(0x7FC0)
        v[b, :, n:] = np.uint16(0x7FC0)
    args = (dev(q), dev(k), dev(v), _i32(lens))
    o, lse = _ops().fa_fwd_kvlen(*args, causal=True, scale=SCALE,
                                 window=window, out_dtype=torch.float32)
    o16, l16 = _ops().fa_fwd_kvlen(*args, causal=True, scale=SCALE,
                                   window=window, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(lse, l16)
    O_ref, L_ref = kvlen_attention(f64(q), f64(k), f64(v), lens, causal=True,
                                   scale=SCALE, window=window)
    compare(host(o), host(lse), O_ref, L_ref, what=f"d{D} kvlen {window}")
