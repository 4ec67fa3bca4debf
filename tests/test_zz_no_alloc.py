"""fa_fwd_noalloc, the entry point that allocates nothing, against fa_fwd
through the C interface: bit-for-bit equal outputs on consecutive calls
that share the library's scratch array (the second call smaller than the
first), for the KV-split form (which uses the scratch) and the prefill
form (which does not), and within the oracle's tolerance."""
import numpy as np
import pytest

from fa_inputs import make_inputs, make_qkv, workload
from oracle import reference_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _both(q, k, v, causal, scale, out_dtype):
    """fa_fwd and fa_fwd_noalloc on the same device inputs, outputs
    pre-filled with NaN."""
    B, Hq, Nq, d = q.shape
    outs = []
    for fn in (_ops().fa_fwd, _ops().fa_fwd_noalloc):
        o = torch.full((B, Hq, Nq, d), float("nan"), dtype=out_dtype,
                       device="cuda")
        lse = torch.full((B, Hq, Nq), float("nan"), device="cuda")
        fn(q, k, v, causal=causal, scale=scale, out_dtype=out_dtype, o=o,
           lse=lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def _check_call(qb, kb, vb, causal, scale, out_dtype, what):
    from exact_io_aware_05_amd import _lib
    B, Hq, Nq, d = qb.shape
    Hkv, Nk = kb.shape[1], kb.shape[2]
    lib = _lib.load()
    splits = lib.fa_default_num_splits(B, Hq, Hkv, Nq, Nk, d)
    (o1, l1), (o2, l2) = _both(dev(qb), dev(kb), dev(vb), causal, scale,
                               out_dtype)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: differs"
    O_ref, L_ref = reference_attention(f64(qb), f64(kb), f64(vb),
                                       causal=causal,
                                       scale=float(np.float32(scale)))
    tol = 1e-2 if out_dtype == torch.float32 else 1.6e-2
    compare(host(o2), host(l2), O_ref, L_ref, o_tol=tol, what=what)
    return splits


def test_noalloc_matches_fa_fwd_on_consecutive_calls():
    # 1) the decode workload (B16 Hq32 Hkv8 Nq1 Nk32768 d128): KV split,
    #    partials in the scratch array
    w = workload(4)
    q, k, v = make_inputs(w, seed=31)
    s1 = _check_call(q, k, v, w.causal, w.scale, torch.float32,
                     "decode workload")
    assert s1 > 1
    # 2) a smaller KV-split call right after it: the scratch keeps the
    #    first call's partials, which must not leak into this one
    q, k, v = make_qkv(2, 8, 2, 3, 3000, 64, seed=32)
    s2 = _check_call(q, k, v, True, 0.125, torch.bfloat16,
                     "small decode after large")
    assert s2 > 1
    # 3) the prefill form (no scratch), then the small decode again
    q, k, v = make_qkv(1, 4, 2, 700, 700, 128, seed=33)
    assert _check_call(q, k, v, True, 128 ** -0.5, torch.float32,
                       "prefill") == 0
    q, k, v = make_qkv(1, 4, 4, 1, 257, 64, seed=34)
    assert _check_call(q, k, v, False, 0.125, torch.float32,
                       "MHA decode after prefill") >= 1
