"""FP8 (E4M3) forward (fa_fwd_fp8) against the float64 oracle on the
decoded inputs: exact where the 8-bit weights are exact (scale 0, rows
with one visible key), and within the tolerance derived from the 8-bit
arithmetic (tests/gpu_util.fp8_tolerance) on random inputs, at small
ragged sizes and at the GQA prefill's full size on sampled rows."""
import numpy as np
import pytest

from fa_inputs import make_fp8
from oracle import decode_e4m3, kv_head_of, reference_attention
from tests.gpu_util import fp8_tolerance, host, FP8_MFMA_REL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _pad_vt(vt8, mult=64):
    """V^T with its key axis padded (zero codes) to a multiple of 64."""
    Nk = vt8.shape[3]
    ldv = (Nk + mult - 1) // mult * mult
    out = np.zeros(vt8.shape[:3] + (ldv,), np.uint8)
    out[..., :Nk] = vt8
    return out


def _run(q8, k8, vt8, qd, kd, vd, causal, scale, out_dtype):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o, lse = _ops().fa_fwd_fp8(t(q8), t(k8), t(_pad_vt(vt8)), t(qd), t(kd),
                               t(vd), causal=causal, scale=scale,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


def _real(q8, k8, vt8, qd, kd, vd):
    q = decode_e4m3(q8) * qd.astype(np.float64)[:, :, None, None]
    k = decode_e4m3(k8) * kd.astype(np.float64)[:, :, None, None]
    v = (decode_e4m3(vt8) * vd.astype(np.float64)[:, :, None, None]
         ).transpose(0, 1, 3, 2)
    return q, k, v


def _check(q8, k8, vt8, qd, kd, vd, causal, scale, rows=None, what=""):
    o32, l32 = _run(q8, k8, vt8, qd, kd, vd, causal, scale, torch.float32)
    o16, l16 = _run(q8, k8, vt8, qd, kd, vd, causal, scale, torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O, L = host(o32), host(l32)
    q, k, v = _real(q8, k8, vt8, qd, kd, vd)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    sc = float(np.float32(scale))
    rows = np.arange(Nq) if rows is None else rows
    worst = 0.0
    for b in range(B):
        O_ref, L_ref, S, P = reference_attention(
            q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=causal, scale=sc,
            rows=rows, return_sp=True)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            # score error bound: 2^-11 of the sum of |q_t k_t| (real units)
            dS = FP8_MFMA_REL * sc * (np.abs(q[b, h, rows]) @ np.abs(k[b, g]).T)
            tol, lse_tol = fp8_tolerance(P[0, h], v[b, g], dS)
            got = O[b, h, rows]
            err = np.abs(got - O_ref[0, h])
            assert np.all(np.isfinite(got)), what
            ratio = float((err / tol).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, (
                f"{what} b{b} h{h}: error {err.max():.3e} beyond the FP8 "
                f"tolerance (ratio {ratio:.2f})")
            fin = np.isfinite(L_ref[0, h])
            np.testing.assert_array_equal(np.isfinite(L[b, h, rows]), fin)
            assert np.all(np.abs(L[b, h, rows][fin] - L_ref[0, h][fin])
                          <= lse_tol[fin]), f"{what} b{b} h{h}: lse"
    print(f"\n{what}: worst error / tolerance = {worst:.3f}")
    return worst


SHAPES = [
    (1, 2, 1, 64, 64, False),
    (1, 4, 2, 300, 300, True),
    (2, 4, 4, 129, 517, False),
    (1, 8, 2, 700, 200, True),    # Nq > Nk: rows that see no key
    (1, 2, 2, 1000, 1000, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:5]))
                         + ("-causal" if s[5] else ""))
def test_fp8_matches_oracle_within_derived_tolerance(shape):
    B, Hq, Hkv, Nq, Nk, causal = shape
    q8, k8, vt8, qd, kd, vd = make_fp8(B, Hq, Hkv, Nq, Nk, 128, seed=51)
    _check(q8, k8, vt8, qd, kd, vd, causal, 1.0 / np.sqrt(128), what=str(shape))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_exact_weights(causal):
    """scale 0: every visible weight is exactly 16 in E4M3, so O is the
    plain mean of the visible V rows (fp32 sums only); causal row 0 sees
    key 0 alone."""
    B, Hq, Hkv, Nq, Nk = 1, 4, 2, 300, 333
    q8, k8, vt8, qd, kd, vd = make_fp8(B, Hq, Hkv, Nq, Nk, 128, seed=52)
    o, lse = _run(q8, k8, vt8, qd, kd, vd, causal, 0.0, torch.float32)
    O = host(o)
    q, k, v = _real(q8, k8, vt8, qd, kd, vd)
    O_ref, L_ref = reference_attention(q, k, v, causal=causal, scale=0.0)
    scale_v = np.abs(v).max()
    assert np.max(np.abs(O - O_ref)) <= 1e-5 * scale_v
    np.testing.assert_allclose(host(lse), L_ref, rtol=0, atol=1e-5)


def test_fp8_gqa_prefill_full_size_sampled_rows():
    """The GQA prefill's shape (B1 Hq32 Hkv8 N8192 d128, causal) in FP8, in
    the benchmark's launch configuration, on sampled rows of every head."""
    q8, k8, vt8, qd, kd, vd = make_fp8(1, 32, 8, 8192, 8192, 128, seed=0)
    rng = np.random.default_rng(53)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 8190, 8191],
                                     rng.choice(8192, size=24, replace=False)]))
    _check(q8, k8, vt8, qd, kd, vd, True, 1.0 / np.sqrt(128), rows=rows,
           what="gqa prefill fp8")
