"""Properties of the HIP path that hold at any size: closed forms, exact
equalities between equivalent calls, determinism, full coverage of the
outputs."""
import math

import numpy as np
import pytest

from fa_inputs import bf16_bits_to_f64, make_qkv, workload
from tests.gpu_util import LSE_TOL, O_TOL, dev, f64, host

pytestmark = pytest.mark.gpu

# different KV split counts of the same call: lse agrees to fp32 rounding
LSE_SPLIT_TOL = 2e-5

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_scale_zero_gives_mean_of_visible_values(causal, d):
    B, Hq, Hkv, N = 1, 4, 2, 333
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=3)
    o, lse = _ops().fa_fwd(dev(q), dev(k), dev(v), causal=causal, scale=0.0,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    vf = f64(v)
    for h in range(Hq):
        vh = vf[0, h // 2]
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(vh, axis=0)[cnt - 1] / cnt[:, None]
        assert np.max(np.abs(O[0, h] - mean)) <= O_TOL
        assert np.max(np.abs(L[0, h] - np.log(cnt))) <= LSE_TOL


def test_gqa_equals_replicated_heads_bitwise():
    B, Hq, Hkv, N, d = 2, 8, 2, 300, 128
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=4)
    rep = Hq // Hkv
    kr, vr = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    for causal in (False, True):
        o1, l1 = _ops().fa_fwd(dev(q), dev(k), dev(v), causal=causal)
        o2, l2 = _ops().fa_fwd(dev(q), dev(kr), dev(vr), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("idx", [1, 3, 4])
def test_deterministic_reruns(idx):
    w = workload(idx).with_(B=min(workload(idx).B, 2))
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, seed=5)
    Q, K, V = dev(q), dev(k), dev(v)
    o1, l1 = _ops().fa_fwd(Q, K, V, causal=w.causal, scale=w.scale)
    o2, l2 = _ops().fa_fwd(Q, K, V, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("idx", [1, 3])
def test_every_output_written(idx):
    """Outputs pre-filled with NaN come back fully finite."""
    w = workload(idx).with_(B=1, Nq=1000, Nk=1000)
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, seed=6)
    o = torch.full((w.B, w.Hq, w.Nq, w.d), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    lse = torch.full((w.B, w.Hq, w.Nq), float("nan"), device="cuda")
    _ops().fa_fwd(dev(q), dev(k), dev(v), causal=w.causal, scale=w.scale,
                  o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_splitkv_every_output_written_and_split_invariant():
    w = workload(4).with_(B=2, Nk=3000)
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, seed=9)
    Q, K, V = dev(q), dev(k), dev(v)
    ref = None
    for S in (1, 2, 7, 94, 200):   # 94 blocks of 32 keys; 200 leaves chunks empty
        o = torch.full((w.B, w.Hq, 1, w.d), float("nan"), dtype=torch.float32,
                       device="cuda")
        lse = torch.full((w.B, w.Hq, 1), float("nan"), device="cuda")
        _ops().fa_fwd_splitkv(Q, K, V, S, scale=w.scale, out_dtype=torch.float32,
                              o=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        if ref is None:
            ref = (o.clone(), lse.clone())
        else:
            # O: chunks differ in the reference max against which each
            # weight is rounded to bf16 (relative 2^-9 per weight), and O is
            # normalised by the sum of those rounded weights.
            assert (o - ref[0]).abs().max().item() <= 2e-3
            # lse comes from the fp32 sums of the unrounded weights, so only
            # fp32 effects remain: the exponent argument s*c2 - m rounded to
            # 2^-24 of |s*c2| + |m| (< 16 here: 6e-7 relative per weight),
            # the per-lane and cross-lane fp32 sums and the merge over at
            # most 200 chunks (< 2^-24 per addition on a chain of < 160:
            # 1e-5 relative), and the 1-ulp exp2 / log2 of the merge.
            assert (lse - ref[1]).abs().max().item() <= LSE_SPLIT_TOL


def test_key_shift_invariance():
    """K' = K + 1 u^T with everything on a coarse grid (exact in bf16):
    O unchanged, lse_i grows by scale * q_i . u."""
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 64
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=10, dist="grid", grid=4)
    u = (np.arange(d) % 5 - 2).astype(np.float32) / 4.0
    kf = bf16_bits_to_f64(k) + u
    from fa_inputs import f32_to_bf16_bits
    k2 = f32_to_bf16_bits(kf.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(k2), kf)       # exact shift
    scale = 0.125
    for causal in (False, True):
        o1, l1 = _ops().fa_fwd(dev(q), dev(k), dev(v), causal=causal,
                               scale=scale, out_dtype=torch.float32)
        o2, l2 = _ops().fa_fwd(dev(q), dev(k2), dev(v), causal=causal,
                               scale=scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        kappa = scale * np.einsum("bhid,d->bhi", bf16_bits_to_f64(q), u)
        assert np.max(np.abs(host(o2) - host(o1))) <= O_TOL
        assert np.max(np.abs(host(l2) - (host(l1) + kappa))) <= LSE_TOL


def test_one_hot_selection():
    """Query i equals key i scaled up: each row selects its own V row."""
    N, d = 256, 64
    c = 18.0
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    for i in range(N):
        q[0, 0, i, i % d] = c
        k[0, 0, i, i % d] = c if i < d else 0.0
    rng = np.random.default_rng(11)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    from fa_inputs import f32_to_bf16_bits
    qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
    o, lse = _ops().fa_fwd(dev(qb), dev(kb), dev(vb), scale=1.0 / 8.0,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    O = host(o)
    vv = f64(vb)
    # rows i < d: key i is the only one aligned with e_i -> O_i = v_i
    assert np.max(np.abs(O[0, 0, :d] - vv[0, 0, :d])) <= O_TOL


def _gqa_prefill_dev(seed, identical_keys=False):
    """The GQA prefill workload's inputs (B1 Hq32 Hkv8 N8192 d128), on the
    device; with ``identical_keys`` every key row of a KV head is the same
    seeded vector."""
    from fa_inputs import f32_to_bf16_bits
    w = workload(3)
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, seed=seed)
    if identical_keys:
        rng = np.random.default_rng(seed + 1)
        row = rng.standard_normal((w.B, w.Hkv, 1, w.d), dtype=np.float32)
        k = f32_to_bf16_bits(np.broadcast_to(row, (w.B, w.Hkv, w.Nk, w.d))
                             .copy())
    return w, q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    """All keys of a KV head equal (scale 1/sqrt(d), not 0): every visible
    key gets the same weight, so O_i is the mean of the visible V rows and
    lse_i = scale q_i.k + ln(#visible).  GQA prefill shape, every row."""
    w, q, k, v = _gqa_prefill_dev(seed=21, identical_keys=True)
    o, lse = _ops().fa_fwd(dev(q), dev(k), dev(v), causal=causal,
                           scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    qf, kf, vf = f64(q), f64(k), f64(v)
    scale = float(np.float32(w.scale))
    G = w.Hq // w.Hkv
    N = w.Nq
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    eo, el = 0.0, 0.0
    for hk in range(w.Hkv):
        csum = np.cumsum(vf[0, hk], axis=0)
        mean = csum[cnt - 1] / cnt[:, None]
        for g in range(G):
            h = hk * G + g
            s = scale * (qf[0, h] @ kf[0, hk, 0])
            eo = max(eo, float(np.max(np.abs(O[0, h] - mean))))
            el = max(el, float(np.max(np.abs(L[0, h] - (s + np.log(cnt))))))
    print(f"\nidentical keys causal={causal}: max|dO|={eo:.3e} "
          f"max|dlse|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("causal", [False, True])
def test_output_rows_in_convex_hull_of_visible_values(causal):
    """Each O_i is a convex combination of the V rows it sees, so every
    coordinate lies between their minimum and maximum.  The fp32 output may
    leave that range only by fp32 rounding of the two sums behind acc / l
    (a few units in the last place); the bf16 output not at all, because
    the bounds are bf16 numbers and rounding to nearest takes a value less
    than half a spacing past a bf16 number back onto it.  GQA prefill
    shape, every row."""
    w, q, k, v = _gqa_prefill_dev(seed=22)
    Q, K, V = dev(q), dev(k), dev(v)
    o32, _ = _ops().fa_fwd(Q, K, V, causal=causal, scale=w.scale,
                           out_dtype=torch.float32)
    o16, _ = _ops().fa_fwd(Q, K, V, causal=causal, scale=w.scale,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    O32, O16 = host(o32), host(o16)
    vf = f64(v)
    G = w.Hq // w.Hkv
    worst = 0.0
    for hk in range(w.Hkv):
        vh = vf[0, hk]
        if causal:
            lo = np.minimum.accumulate(vh, axis=0)
            hi = np.maximum.accumulate(vh, axis=0)
        else:
            lo = np.broadcast_to(vh.min(axis=0), vh.shape)
            hi = np.broadcast_to(vh.max(axis=0), vh.shape)
        for g in range(G):
            h = hk * G + g
            out = np.maximum(lo - O32[0, h], O32[0, h] - hi)
            worst = max(worst, float(out.max()))
            assert np.all(O16[0, h] >= lo) and np.all(O16[0, h] <= hi), \
                f"bf16 O row outside the hull of its visible V rows (h{h})"
    print(f"\nconvex hull causal={causal}: largest excursion of fp32 O "
          f"{worst:.3e}", flush=True)
    assert worst <= 1e-5
