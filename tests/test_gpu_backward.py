"""Parity of the HIP backward pass (through the C interface) with the
float64 oracle of the gradients.

The GPU forward supplies O (bf16) and lse, as in training; the oracle
recomputes everything from the bf16 Q, K, V and dO in float64.  Each
gradient tensor g is graded by max |g - g_ref| <= GRAD_TOL * max |g_ref| +
GRAD_ATOL (tests/gpu_util.py gives the reasoning).
The bf16 gradients must be exactly the round-to-nearest-even bf16 of the
fp32 gradients of the same call."""
import math

import numpy as np
import pytest

from fa_inputs import make_dout, make_inputs, make_qkv, workload
from oracle import reference_attention_backward
from tests.gpu_util import compare_grad, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _gpu_grads(q, k, v, do, causal, scale):
    """fp32 and bf16 gradients of one forward + two backward calls."""
    ops = _ops()
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    o, lse = ops.fa_fwd(Q, K, V, causal=causal, scale=scale)
    g32 = ops.fa_bwd(Q, K, V, o, lse, DO, causal=causal, scale=scale,
                     grad_dtype=torch.float32)
    g16 = ops.fa_bwd(Q, K, V, o, lse, DO, causal=causal, scale=scale,
                     grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for a, b, name in zip(g32, g16, ("dq", "dk", "dv")):
        assert torch.equal(a.to(torch.bfloat16), b), f"bf16 {name} != RNE(fp32)"
    return [host(t) for t in g32]


# B, Hq, Hkv, Nq, Nk, d, causal
SMALL = [
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 1, 17, 17, 64, True),
    (1, 4, 2, 255, 255, 128, True),
    (2, 4, 4, 300, 300, 64, False),
    (1, 8, 1, 200, 500, 128, True),     # MQA, bottom-right causal, Nq < Nk
    (1, 4, 4, 130, 70, 128, True),      # Nq > Nk: rows that see no key
    (1, 2, 2, 128, 128, 128, False),    # exact tile multiples
    (2, 6, 3, 129, 65, 64, False),      # one row / one key past a tile
    (1, 2, 1, 64, 1025, 128, False),
    (1, 4, 1, 700, 33, 64, True),       # many query tiles, one key tile
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_bwd(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=11)
    do = make_dout(B, Hq, Nq, d, seed=11)
    scale = 1.0 / math.sqrt(d)
    got = _gpu_grads(q, k, v, do, causal, scale)
    ref = reference_attention_backward(f64(q), f64(k), f64(v), f64(do),
                                       causal=causal,
                                       scale=float(np.float32(scale)))
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        compare_grad(g, r, what=f"{shape} {name}")
    if causal and Nq > Nk:
        # rows that see no key get no gradient, exactly
        assert np.all(got[0][:, :, :Nq - Nk] == 0.0)


@pytest.mark.parametrize("scale", [0.0, 0.5])
def test_bwd_scale(scale):
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 96, 160, 64
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=12)
    do = make_dout(B, Hq, Nq, d, seed=12)
    got = _gpu_grads(q, k, v, do, True, scale)
    ref = reference_attention_backward(f64(q), f64(k), f64(v), f64(do),
                                       causal=True, scale=scale)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        compare_grad(g, r, what=f"scale {scale} {name}")
    if scale == 0.0:
        # uniform weights carry no gradient into the scores
        assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)


def test_bwd_deterministic():
    q, k, v = make_qkv(1, 4, 2, 333, 333, 128, seed=13)
    do = make_dout(1, 4, 333, 128, seed=13)
    a = _gpu_grads(q, k, v, do, True, 0.1)
    b = _gpu_grads(q, k, v, do, True, 0.1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _workload_bwd(idx, groups):
    """Full-size workload: one forward and the backward over all heads; the
    oracle checks every gradient of the KV heads in ``groups`` (per batch)
    and of the query heads that read them."""
    w = workload(idx)
    q, k, v = make_inputs(w, seed=0)
    do = make_dout(w.B, w.Hq, w.Nq, w.d, seed=0)
    got = _gpu_grads(q, k, v, do, w.causal, w.scale)
    G = w.Hq // w.Hkv
    scale = float(np.float32(w.scale))
    for b in range(w.B):
        for hk in groups:
            hs = slice(hk * G, (hk + 1) * G)
            bs = slice(b, b + 1)
            ref = reference_attention_backward(
                f64(q[bs, hs]), f64(k[bs, hk:hk + 1]), f64(v[bs, hk:hk + 1]),
                f64(do[bs, hs]), causal=w.causal, scale=scale)
            sel = ((bs, hs), (bs, slice(hk, hk + 1)), (bs, slice(hk, hk + 1)))
            for g, r, s, name in zip(got, ref, sel, ("dq", "dk", "dv")):
                e = compare_grad(g[s], r, what=f"{w.name} b{b} kv{hk} {name}")
                print(f"{w.name} b{b} kv{hk} {name}: max err / max |ref| "
                      f"= {e:.2e}")


def test_workload_tiny_bwd():
    _workload_bwd(0, groups=[0])


def test_workload_mha_2048_bwd():
    _workload_bwd(1, groups=[0, 7, 15])


def test_workload_causal_outliers_bwd():
    _workload_bwd(2, groups=[0, 15])


def test_workload_gqa_8192_bwd():
    _workload_bwd(3, groups=[0, 7])
