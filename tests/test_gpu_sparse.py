"""Block-sparse forward (fa_fwd_block_sparse, blocks of 128 query rows x 64
keys) against the float64 oracle with the same block mask: random masks
per head and shared ones, empty mask rows, causal; the two halves of a
query block with very different block lists; the all-ones mask against
fa_fwd bit for bit; and the GQA prefill at full size with a quarter of the
blocks kept, on sampled rows."""
import numpy as np
import pytest

from fa_inputs import make_inputs, make_qkv, workload
from oracle import reference_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
BS = (128, 64)


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _mask(shape, density, seed):
    return (np.random.default_rng(seed).random(shape) < density).astype(np.uint8)


def _nb(N, b):
    return (N + b - 1) // b


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 700, 900, 128), (1, 8, 8, 333, 333, 64),
                                   (1, 2, 1, 300, 2000, 128), (1, 4, 2, 333, 500, 96),
                                   (1, 2, 2, 300, 300, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_random_masks_per_head(shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=81)
    bm = _mask((B, Hq, _nb(Nq, 128), _nb(Nk, 64)), 0.35, seed=82)
    bm[0, 0, 1, :] = 0          # query block 1 of head 0 sees nothing
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_block_sparse(dev(q), dev(k), dev(v),
                                        torch.from_numpy(bm).cuda(),
                                        causal=causal, scale=scale,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale, block_mask=bm,
                                       block_size=BS)
    compare(host(o), host(lse), O_ref, L_ref, what=f"sparse {shape}")


def test_shared_mask_and_bf16_output():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 520, 640, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=83)
    bm = _mask((1, 1, _nb(Nq, 128), _nb(Nk, 64)), 0.5, seed=84)
    M = torch.from_numpy(bm).cuda()
    ops = _ops()
    o32, l32 = ops.fa_fwd_block_sparse(dev(q), dev(k), dev(v), M, causal=True,
                                       out_dtype=torch.float32)
    o16, l16 = ops.fa_fwd_block_sparse(dev(q), dev(k), dev(v), M, causal=True,
                                       out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16) and torch.equal(l32, l16)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=True,
                                       scale=scale, block_mask=bm,
                                       block_size=BS)
    compare(host(o32), host(l32), O_ref, L_ref, what="shared mask")


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_matches_fa_fwd(causal):
    B, Hq, Hkv, N, d = 1, 4, 2, 1000, 128
    q, k, v = make_qkv(B, Hq, Hkv, N, N, d, seed=85)
    M = torch.ones((1, 1, _nb(N, 128), _nb(N, 64)), dtype=torch.uint8,
                   device="cuda")
    ops = _ops()
    a = ops.fa_fwd_block_sparse(dev(q), dev(k), dev(v), M, causal=causal,
                                out_dtype=torch.float32)
    b = ops.fa_fwd(dev(q), dev(k), dev(v), causal=causal,
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_gqa_prefill_quarter_blocks_sampled_rows():
    w = workload(3)
    q, k, v = make_inputs(w, seed=0)
    bm = _mask((1, w.Hq, _nb(w.Nq, 128), _nb(w.Nk, 64)), 0.25, seed=86)
    o, lse = _ops().fa_fwd_block_sparse(dev(q), dev(k), dev(v),
                                        torch.from_numpy(bm).cuda(),
                                        causal=True, scale=w.scale,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = host(o), host(lse)
    del o, lse
    rng = np.random.default_rng(87)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, 8191],
                                     rng.choice(w.Nq, size=30, replace=False)]))
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=True,
                                       scale=float(np.float32(w.scale)),
                                       rows=rows, block_mask=bm, block_size=BS)
    compare(O[:, :, rows], L[:, :, rows], O_ref, L_ref, what="gqa sparse")


@pytest.mark.parametrize("causal", [False, True])
def test_halves_with_unequal_lists(causal):
    """The two 128-row halves of a 256-row query block walk their own block
    lists side by side: one half keeps every key block and the other none,
    or one keeps a single block, or they keep disjoint sets; the half that
    runs out of blocks first still meets every barrier."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 1000, 1200, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=85)
    nqb, nkb = _nb(Nq, 128), _nb(Nk, 64)
    bm = np.zeros((B, Hq, nqb, nkb), dtype=np.uint8)
    bm[0, 0, 0::2, :] = 1          # head 0: even halves all, odd halves none
    bm[0, 1, 0::2, 3] = 1          # head 1: even halves one block ...
    bm[0, 1, 1::2, :] = 1          # ... odd halves all
    bm[0, 2, :, 0::2] = 1          # head 2: disjoint sets per half
    bm[0, 2, 1::2, :] ^= 1
    bm[0, 3] = _mask((nqb, nkb), 0.1, seed=86)[...]
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _ops().fa_fwd_block_sparse(dev(q), dev(k), dev(v),
                                        torch.from_numpy(bm).cuda(),
                                        causal=causal, scale=scale,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = reference_attention(f64(q), f64(k), f64(v), causal=causal,
                                       scale=scale, block_mask=bm,
                                       block_size=BS)
    compare(host(o), host(lse), O_ref, L_ref, what="unequal halves")
