"""Packed variable-length batches through fa_fwd_varlen: every sequence
must match the float64 oracle run on that sequence alone, and a batch of
equal lengths must reproduce fa_fwd on the same rows bit for bit."""
import math

import numpy as np
import pytest

from fa_inputs import make_varlen
from oracle import reference_attention
from tests.gpu_util import compare, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).cuda()


def _run(seqlens_q, seqlens_k, Hq, Hkv, d, causal, out_dtype, seed):
    q, k, v, cu_q, cu_k = make_varlen(seqlens_q, seqlens_k, Hq, Hkv, d,
                                      seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = _ops().fa_fwd_varlen(
        _dev(q), _dev(k), _dev(v), torch.from_numpy(cu_q).cuda(),
        torch.from_numpy(cu_k).cuda(), max(max(seqlens_q), 1),
        max(max(seqlens_k), 1), causal=causal, scale=scale,
        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return q, k, v, cu_q, cu_k, host(o), host(lse), float(np.float32(scale))


# (query lengths, key lengths, Hq, Hkv, d, causal)
CASES = [
    ([17, 300, 1, 256, 511], [17, 300, 1, 256, 511], 4, 2, 128, True),
    ([17, 300, 1, 256, 511], [17, 300, 1, 256, 511], 4, 4, 64, False),
    ([5, 200, 64], [40, 130, 700], 8, 2, 128, True),     # Nq < Nk per sequence
    ([130, 7, 300], [70, 3, 300], 4, 1, 64, True),        # Nq > Nk: empty rows
    ([0, 100, 0, 33], [10, 0, 0, 33], 2, 2, 128, False),  # empty sequences
    ([1000], [1000], 2, 1, 128, True),
    ([17, 300, 1, 256, 511], [17, 300, 1, 256, 511], 4, 2, 96, True),
    ([130, 7, 300], [70, 3, 300], 4, 1, 32, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(
    f"{a}:{b}" for a, b in zip(c[0], c[1])) + f"-h{c[2]}/{c[3]}-d{c[4]}-"
    f"{'causal' if c[5] else 'full'}")
def test_varlen_matches_oracle_per_sequence(case):
    """fp32 output within the forward tolerances of the oracle on every
    sequence; the bf16 output of the same call is the round-to-nearest-even
    of the fp32 one (the kernel rounds only at the store)."""
    lq, lk, Hq, Hkv, d, causal = case
    q, k, v, cu_q, cu_k, O, L, scale = _run(lq, lk, Hq, Hkv, d, causal,
                                            torch.float32, seed=21)
    *_, O16, L16, _ = _run(lq, lk, Hq, Hkv, d, causal, torch.bfloat16,
                           seed=21)
    rne = host(torch.from_numpy(O.astype(np.float32)).to(torch.bfloat16))
    np.testing.assert_array_equal(O16, rne, err_msg="bf16 O != RNE(fp32 O)")
    np.testing.assert_array_equal(L16, L, err_msg="lse depends on out dtype")
    for b in range(len(lq)):
        if lq[b] == 0:
            continue
        rq = slice(cu_q[b], cu_q[b + 1])
        rk = slice(cu_k[b], cu_k[b + 1])
        got_o = O[rq].transpose(1, 0, 2)[None]      # [1, Hq, n, d]
        got_l = L[:, rq][None]                      # [1, Hq, n]
        what = f"sequence {b} ({lq[b]} x {lk[b]})"
        if lk[b] == 0:   # no keys: every row is empty
            assert np.all(got_o == 0.0), what
            assert np.all(np.isneginf(got_l)), what
            continue
        ref_o, ref_l = reference_attention(
            f64(q[rq]).transpose(1, 0, 2)[None],
            f64(k[rk]).transpose(1, 0, 2)[None],
            f64(v[rk]).transpose(1, 0, 2)[None], causal=causal, scale=scale)
        compare(got_o, got_l, ref_o, ref_l, what=what)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_match_fixed_batch(causal):
    B, N, Hq, Hkv, d = 3, 300, 4, 2, 128
    q, k, v, cu_q, cu_k = make_varlen([N] * B, [N] * B, Hq, Hkv, d, seed=22)
    Q, K, V = _dev(q), _dev(k), _dev(v)
    ops = _ops()
    o1, l1 = ops.fa_fwd_varlen(Q, K, V, torch.from_numpy(cu_q).cuda(),
                               torch.from_numpy(cu_k).cuda(), N, N,
                               causal=causal, out_dtype=torch.float32)
    # the same rows as [B, H, N, d]
    to_bhnd = lambda t, H: t.view(B, N, H, d).permute(0, 2, 1, 3).contiguous()
    o2, l2 = ops.fa_fwd(to_bhnd(Q, Hq), to_bhnd(K, Hkv), to_bhnd(V, Hkv),
                        causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(B, N, Hq, d).permute(0, 2, 1, 3), o2)
    assert torch.equal(l1.view(Hq, B, N).permute(1, 0, 2), l2)


def test_varlen_rows_outside_sequences_untouched():
    """Packed rows past cu_seqlens[B] belong to no sequence and keep what
    the caller left there; the covered rows match the full-batch call."""
    q, k, v, cu_q, cu_k = make_varlen([40, 90, 30], [40, 90, 30], 4, 2, 64,
                                      seed=23)
    Q, K, V = _dev(q), _dev(k), _dev(v)
    ops = _ops()
    cq = torch.from_numpy(cu_q[:3].copy()).cuda()   # sequences 0 and 1 only
    ck = torch.from_numpy(cu_k[:3].copy()).cuda()
    o = torch.full((Q.shape[0], 4, 64), 7.0, dtype=torch.float32,
                   device="cuda")
    lse = torch.full((4, Q.shape[0]), 7.0, dtype=torch.float32,
                     device="cuda")
    ops.fa_fwd_varlen(Q, K, V, cq, ck, 90, 90, causal=True,
                      out_dtype=torch.float32, o=o, lse=lse)
    o_all, l_all = ops.fa_fwd_varlen(
        Q, K, V, torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(),
        90, 90, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n = int(cu_q[2])
    assert torch.all(o[n:] == 7.0) and torch.all(lse[:, n:] == 7.0)
    assert torch.equal(o[:n], o_all[:n]) and torch.equal(lse[:, :n],
                                                         l_all[:, :n])
