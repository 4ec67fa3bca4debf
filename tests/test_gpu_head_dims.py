"""Head dimensions 32, 96 and 256 through fa_fwd against the float64 oracle.

32 and 96 run in the prefill kernel's 64- and 128-column tiles with the
columns past d masked (Q and K read as zeros, O not stored); 256 runs in
its own one-wave-per-SIMD prefill kernel when a KV head has many query rows
and in the KV-split form otherwise.  Small and ragged shapes element by
element (both output types, the bf16 one the round-to-nearest-even of the
fp32 one), a GQA prefill of a few thousand rows on every row, outputs
pre-filled with NaN, and strided rows whose padding past d must stay
untouched."""
import numpy as np
import pytest

from fa_inputs import make_qkv
from oracle import reference_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _scale(d):
    return float(np.float32(1.0 / np.sqrt(d)))


# B, Hq, Hkv, Nq, Nk, causal
SHAPES = [
    (1, 1, 1, 1, 1, False),
    (1, 2, 1, 17, 17, True),
    (1, 4, 2, 255, 255, True),
    (2, 6, 3, 129, 65, False),       # one row / one key past a tile
    (1, 8, 1, 300, 700, True),       # MQA, bottom-right causal, Nq < Nk
    (1, 4, 4, 130, 70, True),        # Nq > Nk: fully masked rows
    (1, 2, 2, 256, 128, False),      # exact tile multiples
    (1, 2, 1, 64, 2049, False),
    (2, 8, 2, 1, 3000, False),       # decode rows
    (1, 8, 2, 4, 1500, True),
]


@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fa_fwd_head_dims_match_oracle(shape, d):
    B, Hq, Hkv, Nq, Nk, causal = shape
    print(f"fa_fwd d{d} {shape}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=91)
    Q, K, V = dev(q), dev(k), dev(v)
    scale = _scale(d)
    ops = _ops()
    o32, l32 = ops.fa_fwd(Q, K, V, causal=causal, scale=scale,
                          out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd(Q, K, V, causal=causal, scale=scale,
                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale)
    compare(host(o32), host(l32), O_ref, L_ref, what=f"d{d} {shape}")


# B, Hq, Hkv, N, causal, window: the d = 256 prefill kernel on several
# 128-row query blocks with ragged tails, every row
D256_PREFILL = [
    (1, 8, 4, 2048, True, None),
    (2, 4, 2, 1000, False, None),
    (1, 8, 8, 1500, True, (300, -1)),
    (1, 4, 1, 777, False, (100, 50)),
]


@pytest.mark.parametrize("case", D256_PREFILL,
                         ids=lambda c: "x".join(map(str, c[:5])) + f"-w{c[5]}")
def test_d256_prefill_kernel_every_row(case):
    B, Hq, Hkv, N, causal, window = case
    print(f"d256 prefill {case}", flush=True)
    ops = _ops()
    assert ops.default_num_splits(B, Hq, Hkv, N, N, 256) == 0
    q, k, v = make_qkv(B, Hq, Hkv, N, N, 256, seed=93)
    Q, K, V = dev(q), dev(k), dev(v)
    scale = _scale(256)
    outs = []
    for dt in (torch.float32, torch.bfloat16):
        o = torch.full((B, Hq, N, 256), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((B, Hq, N), float("nan"), device="cuda")
        if window is None:
            ops.fa_fwd(Q, K, V, causal=causal, scale=scale, out_dtype=dt,
                       o=o, lse=lse)
        else:
            ops.fa_fwd_window(Q, K, V, window, causal=causal, scale=scale,
                              out_dtype=dt, o=o, lse=lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o32, l32), (o16, l16) = outs
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale, window=window)
    eo, el = compare(host(o32), host(l32), O_ref, L_ref, what=f"d256 {case}")
    print(f"  max |dO| {eo:.2e}  max |dlse| {el:.2e}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 96])
def test_gqa_prefill_narrow_heads_every_row(d, causal):
    """B1 Hq8 Hkv2 N3000 (several 256-row query blocks and a ragged tail),
    outputs pre-filled with NaN, compared on every row."""
    B, Hq, Hkv, N = 1, 8, 2, 3000
    print(f"gqa prefill d{d} causal={causal}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=92)
    scale = _scale(d)
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32,
                   device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), device="cuda")
    _ops().fa_fwd(dev(q), dev(k), dev(v), causal=causal, scale=scale,
                  out_dtype=torch.float32, o=o, lse=lse)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    for h in range(Hq):
        hk = h // (Hq // Hkv)
        O_ref, L_ref = reference_attention(
            f64(q[:, h:h + 1]), f64(k[:, hk:hk + 1]), f64(v[:, hk:hk + 1]),
            causal=causal, scale=scale)
        compare(O[:, h:h + 1], L[:, h:h + 1], O_ref, L_ref,
                what=f"d{d} head {h}")


@pytest.mark.parametrize("d", [32, 96])
def test_output_row_padding_untouched(d):
    """O rows with a stride past d (the tile's width): the kernel stores
    columns < d only, so the padding keeps its sentinel."""
    B, Hq, Hkv, N = 2, 4, 2, 333
    pad = 64 if d == 32 else 128
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=93)
    Q, K, V = dev(q), dev(k), dev(v)
    scale = _scale(d)
    full = torch.full((B, Hq, N, pad), -7.0, dtype=torch.float32,
                      device="cuda")
    ops = _ops()
    _, lse = ops.fa_fwd_strided(Q, K, V, causal=True, scale=scale,
                                out_dtype=torch.float32, o=full[..., :d])
    ref_o, ref_l = ops.fa_fwd(Q, K, V, causal=True, scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(full[..., d:] == -7.0), "padding past d was written"
    assert torch.equal(full[..., :d], ref_o) and torch.equal(lse, ref_l)
