"""Forward on strided views (fa_fwd_strided): q, k, v sliced out of one
fused QKV projection laid out [B, N, Hq + 2 Hkv, d], O written into a
[B, N, Hq, d] tensor, padded rows; against the float64 oracle on
contiguous copies, and bit for bit against fa_fwd on those copies."""
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


def _fused(q, k, v):
    """[B, N, Hq + 2 Hkv, d] device tensor holding q, k, v (bit patterns
    [B, H, N, d]); returns it and the three [B, H, N, d] views."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    cat = np.concatenate([q, k, v], axis=1).transpose(0, 2, 1, 3)
    T = dev(np.ascontiguousarray(cat))
    Q = T[:, :, :Hq].permute(0, 2, 1, 3)
    K = T[:, :, Hq:Hq + Hkv].permute(0, 2, 1, 3)
    V = T[:, :, Hq + Hkv:].permute(0, 2, 1, 3)
    return T, Q, K, V


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2, 333, 64), (1, 4, 4, 1000, 128),
                                   (2, 4, 2, 333, 96), (1, 4, 4, 300, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fused_qkv_views(shape, causal):
    B, Hq, Hkv, N, d = shape
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=61)
    _, Q, K, V = _fused(q, k, v)
    O_bnhd = torch.empty((B, N, Hq, d), dtype=torch.float32, device="cuda")
    O = O_bnhd.permute(0, 2, 1, 3)
    ops = _ops()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    _, lse = ops.fa_fwd_strided(Q, K, V, causal=causal, scale=scale,
                                out_dtype=torch.float32, o=O)
    ref_o, ref_l = ops.fa_fwd(Q.contiguous(), K.contiguous(), V.contiguous(),
                              causal=causal, scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(O, ref_o) and torch.equal(lse, ref_l)
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale)
    compare(host(O), host(lse), O_ref, L_ref, what=f"fused {shape}")


def test_padded_rows_and_window():
    """K and V rows padded to 136 elements, a sliding window, Nq != Nk."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 200, 700, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=62)
    pad = lambda x: np.concatenate(
        [x, np.full(x.shape[:3] + (8,), 0x7FC0, np.uint16)], axis=3)
    Kp, Vp = dev(pad(k)), dev(pad(v))            # NaN in the padding
    K, V = Kp[..., :d], Vp[..., :d]
    Q = dev(q)
    ops = _ops()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = ops.fa_fwd_strided(Q, K, V, causal=True, window=(90, -1),
                                scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=True,
                                       scale=scale, window=(90, -1))
    compare(host(o), host(lse), O_ref, L_ref, what="padded rows")
