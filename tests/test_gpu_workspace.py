"""The KV-split form inside fa_fwd keeps one workspace per (device, stream)
and grows it on demand.  Calls of growing and shrinking size on two streams
running at once must each give exactly what fa_fwd_splitkv gives with a
workspace of its own (same split count, same kernels)."""
import numpy as np
import pytest

from fa_inputs import make_qkv
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ops():
    from exact_io_aware_05_amd import ops
    return ops


# decode shapes (one query per sequence): the KV-split form
SHAPES = [(2, 8, 2, 1, 4096, 128), (2, 8, 2, 1, 16384, 128),
          (1, 16, 4, 2, 2048, 64), (3, 8, 2, 1, 9000, 128),
          (2, 8, 2, 1, 700, 128)]


def test_fa_fwd_workspace_per_stream():
    ops = _ops()
    cases = []
    for i, (B, Hq, Hkv, Nq, Nk, d) in enumerate(SHAPES):
        assert ops.default_num_splits(B, Hq, Hkv, Nq, Nk, d) > 0
        q, k, v = make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=90 + i)
        cases.append((dev(q), dev(k), dev(v)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = [[None] * len(cases) for _ in streams]
    # three rounds, every case on both streams, no synchronisation between
    # the streams inside a round
    for _ in range(3):
        for i, (q, k, v) in enumerate(cases):
            for si, st in enumerate(streams):
                with torch.cuda.stream(st):
                    outs[si][i] = ops.fa_fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, ((q, k, v), shp) in enumerate(zip(cases, SHAPES)):
        B, Hq, Hkv, Nq, Nk, d = shp
        splits = ops.default_num_splits(B, Hq, Hkv, Nq, Nk, d)
        o_ref, l_ref = ops.fa_fwd_splitkv(q, k, v, splits,
                                          out_dtype=torch.float32)
        torch.cuda.synchronize()
        for si in range(len(streams)):
            o, lse = outs[si][i]
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), \
                (shp, si)


def test_fa_fwd_kvsplit_under_graph_capture():
    """Under stream capture the KV-split form takes its workspace with
    hipMallocAsync / hipFreeAsync on the stream (memory the graph owns), not
    the per-stream buffer.  Replays, with eager calls of another size on the
    same stream between them, match the eager result bit for bit."""
    ops = _ops()
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 1, 4096, 128
    q, k, v = (dev(x) for x in make_qkv(B, Hq, Hkv, Nq, Nk, d, seed=97))
    q2, k2, v2 = (dev(x) for x in make_qkv(1, 16, 4, 1, 9000, 128, seed=98))
    o_ref, l_ref = ops.fa_fwd(q, k, v, out_dtype=torch.float32)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.fa_fwd(q, k, v, out_dtype=torch.float32, o=o, lse=lse)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
        with torch.cuda.stream(s):
            ops.fa_fwd(q2, k2, v2, out_dtype=torch.float32)
        torch.cuda.synchronize()
