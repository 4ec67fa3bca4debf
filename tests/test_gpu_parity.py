"""Parity of the HIP path (through the C interface) with the float64 oracle.

Small and ragged shapes are compared element by element against the full
oracle; the five workloads run at their full sizes in the launch
configuration the benchmark times, with the outputs pre-filled with NaN,
and are compared on every output element (every query row of every head)."""
import math

import numpy as np
import pytest

from fa_inputs import make_inputs, make_qkv, workload
from oracle import reference_attention
from tests.gpu_util import LSE_TOL, O_TOL, compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(fn, q, k, v, **kw):
    o, lse = fn(dev(q), dev(k), dev(v), **kw)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _fa():
    from exact_io_aware_05_amd import ops
    return ops


# B, Hq, Hkv, Nq, Nk, d, causal
SMALL = [
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 1, 17, 17, 64, True),
    (1, 4, 2, 255, 255, 128, True),
    (2, 4, 4, 1000, 1000, 64, False),
    (1, 8, 1, 300, 700, 128, True),     # MQA, bottom-right causal, Nq < Nk
    (1, 4, 4, 130, 70, 128, True),      # Nq > Nk: fully masked rows
    (1, 2, 2, 128, 128, 128, False),    # exact tile multiples
    (2, 6, 3, 129, 65, 64, False),      # one row / one key past a tile
    (1, 2, 1, 64, 2049, 128, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_small_shapes_fa_fwd(shape, out):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=7)
    scale = 1.0 / math.sqrt(d)
    od = torch.float32 if out == "f32" else torch.bfloat16
    O, lse = _run(_fa().fa_fwd, q, k, v, causal=causal, scale=scale,
                  out_dtype=od)
    O_ref, lse_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                         scale=float(np.float32(scale)))
    compare(O, lse, O_ref, lse_ref, what=str(shape))


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_small_shapes_splitkv(shape, splits):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=8)
    scale = 1.0 / math.sqrt(d)
    O, lse = _run(_fa().fa_fwd_splitkv, q, k, v, num_splits=splits,
                  causal=causal, scale=scale, out_dtype=torch.float32)
    O_ref, lse_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                         scale=float(np.float32(scale)))
    compare(O, lse, O_ref, lse_ref, what=f"{shape} S={splits}")


def _sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(rows))


def _bf16_half_ulp(x):
    """Half the spacing of bf16 numbers around |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def _workload_parity(idx, sample=None, seed=0):
    """Full-size workload in the benchmark's launch configuration.

    Accuracy is graded on the fp32 output of the kernel (max-abs 1e-2 on O,
    1e-3 on lse).  The bf16 output of the same call must be exactly the
    round-to-nearest-even bf16 of that fp32 output, and its distance to the
    oracle is then bounded by the tolerance plus half a bf16 spacing (bf16
    cannot hold |O| >= 4 closer than 2^-6).  Both outputs start as NaN, so
    an element the kernel never writes fails.  The oracle runs one head at
    a time (``sample``: only some query rows, for quick local runs)."""
    w = workload(idx)
    q, k, v = make_inputs(w, seed=seed)
    Q, K, V = dev(q), dev(k), dev(v)

    def nan_out(dtype):
        return (torch.full((w.B, w.Hq, w.Nq, w.d), float("nan"), dtype=dtype,
                           device="cuda"),
                torch.full((w.B, w.Hq, w.Nq), float("nan"), device="cuda"))

    o32, lse32 = nan_out(torch.float32)
    o16, lse16 = nan_out(torch.bfloat16)
    _fa().fa_fwd(Q, K, V, causal=w.causal, scale=w.scale,
                 out_dtype=torch.float32, o=o32, lse=lse32)
    _fa().fa_fwd(Q, K, V, causal=w.causal, scale=w.scale,
                 out_dtype=torch.bfloat16, o=o16, lse=lse16)
    torch.cuda.synchronize()
    assert not torch.isnan(o32).any() and not torch.isnan(lse32).any(), \
        "unwritten output elements"
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(lse32, lse16)
    O32, O16, L = host(o32), host(o16), host(lse32)
    del o32, o16, lse32, lse16
    scale = float(np.float32(w.scale))
    rows = None if sample is None else _sample_rows(w.Nq, sample, seed=idx)
    G = w.Hq // w.Hkv
    e32, e16, el = 0.0, 0.0, 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // G
            O_ref, L_ref = reference_attention(
                f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, hk:hk + 1]),
                f64(v[b:b + 1, hk:hk + 1]), causal=w.causal, scale=scale,
                rows=rows)
            sel = (slice(b, b + 1), slice(h, h + 1),
                   slice(None) if rows is None else rows)
            eo, eb = compare(O32[sel], L[sel], O_ref, L_ref, O_TOL, LSE_TOL,
                             f"{w.name} b{b} h{h} fp32 O")
            d16 = np.abs(O16[sel] - O_ref)
            bound = O_TOL + _bf16_half_ulp(O_ref)
            assert np.all(d16 <= bound), f"{w.name} b{b} h{h}: bf16 O beyond bound"
            e32, el = max(e32, eo), max(el, eb)
            e16 = max(e16, float(d16.max()))
    print(f"\n{w.name}: {'all' if rows is None else len(rows)} rows x "
          f"{w.B * w.Hq} heads: max|dO| fp32-out={e32:.3e} "
          f"bf16-out={e16:.3e} max|dlse|={el:.3e}", flush=True)
    return e32, e16, el


def test_workload_tiny():
    _workload_parity(0)


def test_workload_mha_d64():
    _workload_parity(1)


def test_workload_causal_outliers():
    _workload_parity(2)


def test_workload_gqa_prefill():
    _workload_parity(3)


def test_workload_decode():
    _workload_parity(4)


def _scaled_keys(B, H, N, d, seed, lo, hi, factor):
    """Seeded N(0,1) Q/K/V with the keys lo..hi-1 scaled by `factor`
    (before the bf16 rounding), so the scores jump between K/V blocks."""
    from fa_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k[:, :, lo:hi, :] *= np.float32(factor)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


@pytest.mark.parametrize("pattern", ["grow", "shrink"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_scores_jumping_between_blocks(pattern, causal, d):
    """Scores that grow (or fall) by far more than any reference-max
    threshold from one K/V block to the next: the running max must move and
    the accumulated output be rescaled (or later weights underflow)."""
    N = 400
    lo, hi = (130, N) if pattern == "grow" else (0, 70)
    q, k, v = _scaled_keys(1, 2, N, d, seed=11, lo=lo, hi=hi, factor=40.0)
    scale = 1.0 / math.sqrt(d)
    O, L = _run(_fa().fa_fwd, q, k, v, causal=causal, scale=scale,
                out_dtype=torch.float32)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=float(np.float32(scale)))
    compare(O, L, O_ref, L_ref, what=f"jump {pattern} d{d} causal={causal}")
