"""The prefill form of the paged and padded-cache entry points: query chunks
of many rows over a paged KV cache (fa_fwd_paged) or over a padded cache
with per-sequence lengths (fa_fwd_kvlen) run on the tiled prefill kernel.

Against the float64 oracles: several 256-row query tiles with ragged tails,
sequences shorter and longer than the chunk (causal rows that see no key),
empty sequences, GQA, no mask / causal / sliding window, page sizes 64 to
256, d = 32, 64, 96 and 128.  Pool rows that belong to no sequence, and the
rows past each sequence's length, hold NaN (reading one would show), and
page-table entries past a sequence's pages hold garbage.  Outputs are
pre-filled with NaN so that a row left unwritten shows too.

And bit for bit: the kernel's arithmetic does not depend on where a block
lives, so a paged call equals fa_fwd on the same rows gathered into a
contiguous cache, and a padded call at full lengths equals fa_fwd."""
import numpy as np
import pytest

from fa_inputs import make_paged, make_qkv
from oracle import kvlen_attention, paged_attention
from tests.gpu_util import compare, dev, f64, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAN_BF16 = np.uint16(0x7FC0)


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _poisoned_paged(B, Hq, Hkv, Nq, d, P, maxp, lens, seed):
    """make_paged, then NaN in every pool row that no sequence uses and
    garbage in the table entries past each sequence's pages."""
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, d, P, maxp, lens,
                                      seed=seed)
    kc, vc, table = kc.copy(), vc.copy(), table.copy()
    used = np.zeros(kc.shape[:2], dtype=bool)
    for b, n in enumerate(lens):
        for r in range(n):
            used[table[b, r // P], r % P] = True
        npg = (n + P - 1) // P
        table[b, npg:] = np.where(np.arange(maxp - npg) % 2, -7, 1 << 30)
    kc[~used] = NAN_BF16
    vc[~used] = NAN_BF16
    return q, kc, vc, table, sl


def _nan_out(B, Hq, Nq, d, dtype):
    o = torch.full((B, Hq, Nq, d), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32,
                     device="cuda")
    return o, lse


# B, Hq, Hkv, Nq, d, page_size, max_pages, seqlens, causal, window
PAGED_CASES = [
    (2, 8, 2, 600, 128, 64, 12, [700, 300], True, (-1, -1)),
    (3, 4, 4, 300, 64, 128, 8, [1000, 0, 513], False, (-1, -1)),
    (2, 8, 2, 513, 96, 64, 10, [640, 513], True, (-1, -1)),
    (2, 4, 1, 257, 32, 256, 4, [900, 100], True, (-1, -1)),
    (2, 16, 4, 300, 128, 128, 10, [1200, 299], False, (200, 0)),
    (1, 8, 8, 800, 64, 64, 20, [1250], True, (333, -1)),
]


def _paged_id(c):
    return (f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}d{c[4]}p{c[5]}x{c[6]}"
            f"{'-causal' if c[8] else ''}-w{c[9][0]},{c[9][1]}")


@pytest.mark.parametrize("case", PAGED_CASES, ids=_paged_id)
def test_paged_prefill_matches_oracle(case):
    B, Hq, Hkv, Nq, d, P, maxp, lens, causal, window = case
    print(f"paged prefill case {case}", flush=True)
    ops = _ops()
    assert ops.paged_num_splits(B, Hq, Hkv, Nq, d, P, maxp) == 0, \
        "expected the prefill form"
    q, kc, vc, table, sl = _poisoned_paged(B, Hq, Hkv, Nq, d, P, maxp, lens,
                                           seed=61)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    args = (dev(q), dev(kc), dev(vc), _i32(table), _i32(sl))
    o32, l32 = _nan_out(B, Hq, Nq, d, torch.float32)
    o16, l16 = _nan_out(B, Hq, Nq, d, torch.bfloat16)
    ops.fa_fwd_paged(*args, causal=causal, scale=scale, window=window,
                     out_dtype=torch.float32, o=o32, lse=l32)
    ops.fa_fwd_paged(*args, causal=causal, scale=scale, window=window,
                     out_dtype=torch.bfloat16, o=o16, lse=l16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = paged_attention(f64(q), f64(kc), f64(vc), table, sl,
                                   causal=causal, scale=scale, window=window)
    eo, el = compare(host(o32), host(l32), O_ref, L_ref,
                     what=f"paged prefill {case}")
    print(f"  max |dO| {eo:.2e}  max |dlse| {el:.2e}", flush=True)


@pytest.mark.parametrize("window", [(-1, -1), (-1, 0), (1000, 0)],
                         ids=["none", "causal", "window1000"])
def test_paged_prefill_equals_fa_fwd_on_gathered_rows(window):
    """Scattered 256-key pages against the same rows in a contiguous cache,
    bit for bit, at a chunk of 2048 queries at the end of a 4096-key cache
    (GQA 32/8, d = 128)."""
    B, Hq, Hkv, Nq, d, P, maxp = 1, 32, 8, 2048, 128, 256, 16
    N = P * maxp
    print(f"paged prefill vs fa_fwd window {window}", flush=True)
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, d, P, maxp, [N] * B,
                                      seed=62)
    ops = _ops()
    assert ops.paged_num_splits(B, Hq, Hkv, Nq, d, P, maxp) == 0
    kcd, vcd, td = dev(kc), dev(vc), _i32(table)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o1, l1 = ops.fa_fwd_paged(dev(q), kcd, vcd, td, _i32(sl), scale=scale,
                              window=window, out_dtype=torch.float32)
    # the sequence's rows in order: [B, Hkv, N, d]
    k = kcd[td.long()].reshape(B, N, Hkv, d).permute(0, 2, 1, 3).contiguous()
    v = vcd[td.long()].reshape(B, N, Hkv, d).permute(0, 2, 1, 3).contiguous()
    o2, l2 = ops.fa_fwd_window(dev(q), k, v, window=window, scale=scale,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# B, Hq, Hkv, Nq, Nk (padded), d, lengths, causal, window
KVLEN_CASES = [
    (3, 8, 2, 600, 900, 128, [900, 0, 455], True, (-1, -1)),
    (2, 4, 4, 300, 640, 64, [640, 257], False, (-1, -1)),
    (2, 8, 2, 400, 512, 96, [512, 300], True, (-1, -1)),
    (2, 8, 8, 260, 700, 32, [700, 65], False, (128, 64)),
    (2, 8, 4, 300, 700, 256, [700, 333], True, (-1, -1)),
]


@pytest.mark.parametrize("case", KVLEN_CASES, ids=lambda c: (
    f"B{c[0]}h{c[1]}/{c[2]}q{c[3]}k{c[4]}d{c[5]}"
    f"{'-causal' if c[7] else ''}-w{c[8][0]},{c[8][1]}"))
def test_kvlen_prefill_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, lens, causal, window = case
    print(f"kvlen prefill case {case}", flush=True)
    ops = _ops()
    assert ops.default_num_splits(B, Hq, Hkv, Nq, Nk, d) == 0
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=63)
    k, v = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k[b, :, n:] = NAN_BF16
        v[b, :, n:] = NAN_BF16
    scale = float(np.float32(1.0 / np.sqrt(d)))
    args = (dev(q), dev(k), dev(v), _i32(lens))
    o32, l32 = _nan_out(B, Hq, Nq, d, torch.float32)
    o16, l16 = _nan_out(B, Hq, Nq, d, torch.bfloat16)
    ops.fa_fwd_kvlen(*args, causal=causal, scale=scale, window=window,
                     out_dtype=torch.float32, o=o32, lse=l32)
    ops.fa_fwd_kvlen(*args, causal=causal, scale=scale, window=window,
                     out_dtype=torch.bfloat16, o=o16, lse=l16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 O != RNE(fp32 O)"
    assert torch.equal(l32, l16)
    O_ref, L_ref = kvlen_attention(f64(q), f64(k), f64(v), lens,
                                   causal=causal, scale=scale, window=window)
    eo, el = compare(host(o32), host(l32), O_ref, L_ref,
                     what=f"kvlen prefill {case}")
    print(f"  max |dO| {eo:.2e}  max |dlse| {el:.2e}", flush=True)


def test_kvlen_prefill_full_lengths_equal_fa_fwd():
    B, Hq, Hkv, Nq, Nk, d = 2, 16, 4, 1000, 1500, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=64)
    ops = _ops()
    o1, l1 = ops.fa_fwd_kvlen(dev(q), dev(k), dev(v), _i32([Nk] * B),
                              causal=True, out_dtype=torch.float32)
    o2, l2 = ops.fa_fwd(dev(q), dev(k), dev(v), causal=True,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_small_pages_many_rows_take_the_kvsplit_form():
    """32-key pages cannot hold the prefill kernel's 64-key blocks, so a
    chunk of many queries over them runs the KV-split form (many packed row
    tiles per KV head); the result is the same attention."""
    B, Hq, Hkv, Nq, d, P, maxp = 2, 8, 2, 300, 128, 32, 24
    lens = [700, 301]
    print("paged small pages, many rows", flush=True)
    ops = _ops()
    assert ops.paged_num_splits(B, Hq, Hkv, Nq, d, P, maxp) >= 1
    q, kc, vc, table, sl = _poisoned_paged(B, Hq, Hkv, Nq, d, P, maxp, lens,
                                           seed=65)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _nan_out(B, Hq, Nq, d, torch.float32)
    ops.fa_fwd_paged(dev(q), dev(kc), dev(vc), _i32(table), _i32(sl),
                     causal=True, scale=scale, out_dtype=torch.float32,
                     o=o, lse=lse)
    torch.cuda.synchronize()
    O_ref, L_ref = paged_attention(f64(q), f64(kc), f64(vc), table, sl,
                                   causal=True, scale=scale)
    compare(host(o), host(lse), O_ref, L_ref, what="paged 32-key pages")
