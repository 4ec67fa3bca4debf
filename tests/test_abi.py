"""The C interface on the host: the library loads without a GPU, exports
every function the header declares, and rejects bad arguments with the
documented status codes before touching the GPU (no compute call here)."""
import ctypes
import threading
import math
import os
import re
import subprocess
import sys

import pytest

from exact_io_aware_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()



def _fresh(call):
    """Run ``call`` on a new thread and return its result: a call that gets
    as far as the device query (FA_ERR_HIP on this host) then leaves the
    per-thread last HIP error of the test thread untouched."""
    out = []
    t = threading.Thread(target=lambda: out.append(call()))
    t.start()
    t.join()
    return out[0]

def test_header_declares_the_interface():
    assert _declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(fa_[a-z0-9_]+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code, word in ((0, b"FA_OK"), (1, b"INVALID"), (2, b"UNSUPPORTED"),
                       (3, b"HIP")):
        assert word in lib.fa_status_string(code)
    assert lib.fa_status_string(99) == b"unknown fa status"


# fake but aligned, non-null "device" pointers: validation must fail first
P = 0x10000


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=64,
             causal=0, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                      a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                      a["scale"], a["out"], None)


def _split(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=1, Nk=64, d=64,
             causal=0, scale=0.125, out=0, S=2, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                              a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                              a["causal"], a["scale"], a["out"], a["S"],
                              a["ws"], a["wsb"], None)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(q=P + 8), dict(k=P + 2), dict(v=P + 4), dict(o=P + 1), dict(lse=P + 2),
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nk=0), dict(d=0),
    dict(B=-1), dict(Hq=6, Hkv=4), dict(scale=math.nan), dict(scale=math.inf),
    dict(scale=-0.5), dict(out=2), dict(out=-1),
]


@pytest.mark.parametrize("kw", INVALID, ids=lambda k: str(k))
def test_fwd_invalid_arguments(lib, kw):
    assert _fwd(lib, **kw) == _lib.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [16, 48, 100, 160, 512])
def test_fwd_unsupported_head_dim(lib, d):
    assert _fwd(lib, d=d) == _lib.FA_ERR_UNSUPPORTED


# On this host (no GPU) a call whose arguments pass every check stops at the
# device query with FA_ERR_HIP: that is how a supported head dimension shows.
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_fwd_head_dims_pass_validation(lib, d):
    assert _fresh(lambda: _fwd(lib, d=d)) == _lib.FA_ERR_HIP
    assert _fresh(lambda: _fwd(lib, d=d, Nq=1, Nk=4096)) == _lib.FA_ERR_HIP
    assert _fresh(lambda: lib.fa_fwd_noalloc(P, P, P, P, P, 1, 4, 2, 16, 16, d,
                                             0, 0.125, 0, None)) == \
        _lib.FA_ERR_HIP


def test_fwd_form_by_head_dim(lib):
    """fa_fwd's form: d = 96 always runs the prefill kernel (0 chunks); d =
    256 takes the prefill form (its own kernel) for many query rows per KV
    head and the KV-split form for few, like d = 64 and 128."""
    assert lib.fa_default_num_splits(1, 32, 8, 8192, 8192, 128) == 0
    assert lib.fa_default_num_splits(1, 32, 8, 1, 8192, 128) > 1
    assert lib.fa_default_num_splits(1, 32, 8, 8192, 8192, 96) == 0
    assert lib.fa_default_num_splits(1, 32, 8, 1, 8192, 96) == 0
    assert lib.fa_default_num_splits(1, 32, 8, 8192, 8192, 256) == 0
    assert lib.fa_default_num_splits(1, 32, 8, 1, 8192, 256) > 1
    assert lib.fa_default_num_splits(1, 32, 8, 1, 8192, 100) == 0


def test_fwd_prefill_kv_head_range(lib):
    # one K/V head of the prefill form must span < 2^31 bytes; the refusal
    # comes before any HIP call (the last HIP error is per thread, so a
    # fresh thread starts from 0)
    out = {}

    def calls():
        out["a"] = _fwd(lib, Hq=1, Hkv=1, Nq=4096, Nk=1 << 23, d=128)
        out["b"] = _fwd(lib, Hq=1, Hkv=1, Nq=4096, Nk=1 << 24, d=64)
        out["hip"] = lib.fa_last_hip_error()

    t = threading.Thread(target=calls)
    t.start()
    t.join()
    assert out == {"a": _lib.FA_ERR_UNSUPPORTED, "b": _lib.FA_ERR_UNSUPPORTED,
                   "hip": 0}


@pytest.mark.parametrize("kw", INVALID + [dict(S=0), dict(S=5000), dict(ws=None),
                                          dict(ws=P + 4), dict(wsb=16)],
                         ids=lambda k: str(k))
def test_splitkv_invalid_arguments(lib, kw):
    assert _split(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_splitkv_kv_head_range(lib):
    # one K/V head must span < 2^31 bytes in the KV-split form too
    assert _split(lib, Hq=1, Hkv=1, Nq=1, Nk=1 << 23, d=128, S=1,
                  wsb=1 << 20) == _lib.FA_ERR_UNSUPPORTED
    assert _fwd(lib, Hq=1, Hkv=1, Nq=1, Nk=1 << 23, d=128) == \
        _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def test_splitkv_workspace_size(lib):
    # rows * splits * (d fp32 partial outputs + (m, l, lb, unused) fp32)
    assert lib.fa_splitkv_workspace_bytes(16, 32, 1, 128, 16) == \
        16 * 32 * 16 * (128 * 4 + 16)
    assert lib.fa_splitkv_workspace_bytes(1, 1, 1, 64, 1) == 64 * 4 + 16
    assert lib.fa_splitkv_workspace_bytes(0, 1, 1, 64, 1) == 0
    assert lib.fa_splitkv_workspace_bytes(1, 1, 1, 64, 0) == 0


def test_default_split_choice(lib):
    # single-query decode over a 32K cache, 128 (batch, KV head) pairs:
    # one wave per SIMD (1024 waves)
    assert lib.fa_default_num_splits(16, 32, 8, 1, 32768, 128) == 8
    # prefill shapes use the tiled kernel
    assert lib.fa_default_num_splits(1, 32, 8, 8192, 8192, 128) == 0
    assert lib.fa_default_num_splits(4, 16, 16, 2048, 2048, 64) == 0
    # small caches get at most one chunk per 4 blocks of 32 keys
    assert lib.fa_default_num_splits(1, 1, 1, 1, 64, 64) == 1
    assert lib.fa_default_num_splits(1, 1, 1, 1, 4096, 64) == 32
    # invalid sizes give 0
    assert lib.fa_default_num_splits(1, 3, 2, 1, 64, 64) == 0
    assert lib.fa_default_num_splits(1, 1, 1, 1, 64, 80) == 0


def _bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4,
             Hkv=2, Nq=16, Nk=16, d=64, causal=0, scale=0.125, out=0, ws=P,
             wsb=1 << 20)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                      a["dq"], a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"],
                      a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                      a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize(
    "kw", INVALID + [dict(do=None), dict(dq=None), dict(dk=None), dict(dv=None),
                     dict(do=P + 8), dict(dq=P + 2), dict(dk=P + 4),
                     dict(dv=P + 1), dict(ws=None), dict(ws=P + 4),
                     dict(wsb=4 * 16 * 8 - 1)],
    ids=lambda k: str(k))
def test_bwd_invalid_arguments(lib, kw):
    assert _bwd(lib, **kw) == _lib.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [32, 96, 256])
def test_bwd_unsupported_head_dim(lib, d):
    assert _bwd(lib, d=d) == _lib.FA_ERR_UNSUPPORTED


def test_bwd_head_range(lib):
    # one head of Q (or K) plus one 128-row step must span < 2^31 bytes
    big = (1 << 23) - 128
    assert _bwd(lib, Hq=1, Hkv=1, Nq=big + 1, Nk=16, d=128,
                wsb=1 << 40) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd(lib, Hq=1, Hkv=1, Nq=16, Nk=big + 1, d=128) == \
        _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def test_bwd_workspace_size(lib):
    # D and lse * log2(e): two fp32 per query row
    assert lib.fa_bwd_workspace_bytes(1, 32, 8192) == 32 * 8192 * 8
    assert lib.fa_bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 8
    assert lib.fa_bwd_workspace_bytes(0, 1, 1) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 0) == 0


def _varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=2, Hq=4, Hkv=2, tq=32,
             tk=40, mq=16, mk=20, d=64, causal=0, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"],
                             a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"],
                             a["tq"], a["tk"], a["mq"], a["mk"], a["d"],
                             a["causal"], a["scale"], a["out"], None)


@pytest.mark.parametrize(
    "kw", [dict(q=None), dict(k=P + 8), dict(o=P + 1), dict(lse=P + 2),
           dict(cq=None), dict(ck=None), dict(cq=P + 2), dict(ck=P + 1),
           dict(B=0), dict(Hq=6, Hkv=4), dict(tq=0), dict(tk=0), dict(mq=0),
           dict(mk=0), dict(scale=math.nan), dict(out=3)],
    ids=lambda k: str(k))
def test_varlen_invalid_arguments(lib, kw):
    assert _varlen(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_varlen_unsupported(lib):
    assert _varlen(lib, d=256) == _lib.FA_ERR_UNSUPPORTED
    assert _varlen(lib, d=100) == _lib.FA_ERR_UNSUPPORTED
    assert _fresh(lambda: _varlen(lib, d=96)) == _lib.FA_ERR_HIP
    assert _fresh(lambda: _varlen(lib, d=32)) == _lib.FA_ERR_HIP
    # one sequence's K/V rows of one head span (mk - 1) * Hkv * d * 2 + 2d
    assert _varlen(lib, Hkv=8, Hq=8, mk=(1 << 20) + 2, d=128) == \
        _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def test_no_hip_error_recorded_by_validation(lib):
    _fwd(lib, q=None)
    _split(lib, S=0)
    _bwd(lib, ws=None)
    assert lib.fa_last_hip_error() == 0


def _win(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=64,
             causal=0, wl=4, wr=0, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                             a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                             a["causal"], a["wl"], a["wr"], a["scale"],
                             a["out"], None)


@pytest.mark.parametrize("kw", INVALID + [dict(wl=-2), dict(wr=-2),
                                          dict(wl=-5, wr=3)],
                         ids=lambda k: str(k))
def test_window_invalid_arguments(lib, kw):
    assert _win(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_window_unsupported(lib):
    assert _win(lib, d=100) == _lib.FA_ERR_UNSUPPORTED
    assert _win(lib, d=100, wl=-1, wr=-1) == _lib.FA_ERR_UNSUPPORTED
    for d in (32, 96, 256):
        assert _fresh(lambda: _win(lib, d=d)) == _lib.FA_ERR_HIP
    assert _win(lib, Nk=(1 << 23) + 1, d=128) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def _bwdw(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4,
             Hkv=2, Nq=16, Nk=16, d=64, causal=0, wl=4, wr=0, scale=0.125,
             out=0, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.fa_bwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"],
                             a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                             a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                             a["causal"], a["wl"], a["wr"], a["scale"],
                             a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw", INVALID + [dict(wl=-2), dict(wr=-3),
                                          dict(do=None), dict(dq=P + 4),
                                          dict(ws=None), dict(wsb=8)],
                         ids=lambda k: str(k))
def test_bwd_window_invalid_arguments(lib, kw):
    assert _bwdw(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_bwd_window_unsupported(lib):
    assert _bwdw(lib, d=96) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def _paged(lib, **kw):
    a = dict(q=P, kc=P, vc=P, o=P, lse=P, pt=P, sl=P, B=2, Hq=4, Hkv=2, Nq=1,
             d=64, np_=16, ps=32, mp=8, causal=0, wl=-1, wr=-1, scale=0.125,
             out=0, S=0, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.fa_fwd_paged(a["q"], a["kc"], a["vc"], a["o"], a["lse"],
                            a["pt"], a["sl"], a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["d"], a["np_"], a["ps"], a["mp"],
                            a["causal"], a["wl"], a["wr"], a["scale"],
                            a["out"], a["S"], a["ws"], a["wsb"], None)


PAGED_INVALID = [
    dict(q=None), dict(kc=P + 2), dict(vc=None), dict(o=P + 4), dict(lse=None),
    dict(pt=None), dict(sl=None), dict(pt=P + 2), dict(sl=P + 1),
    dict(B=0), dict(Hq=3), dict(Nq=0), dict(np_=0), dict(mp=0),
    dict(ps=16), dict(ps=48), dict(ps=0), dict(wl=-2), dict(wr=-7),
    dict(scale=-1.0), dict(out=5), dict(S=-1), dict(S=4097),
    dict(ws=None), dict(ws=P + 8), dict(wsb=0),
    # a 32-page chunk limit: 32-key pages, 1000 pages per sequence need >= 17
    dict(mp=1000, S=16),
]


@pytest.mark.parametrize("kw", PAGED_INVALID, ids=lambda k: str(k))
def test_paged_invalid_arguments(lib, kw):
    assert _paged(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_paged_unsupported_and_splits(lib):
    # d = 96 runs only in the prefill form: not with 32-key pages, not with
    # an explicit split count
    assert _paged(lib, d=96) == _lib.FA_ERR_UNSUPPORTED
    assert _paged(lib, d=96, ps=64, Nq=100, S=2) == _lib.FA_ERR_UNSUPPORTED
    assert _paged(lib, ps=1 << 16, mp=1 << 15) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0
    # default split count: at least one chunk, none over 62 pages
    assert lib.fa_paged_num_splits(1, 4, 2, 1, 64, 32, 1000) >= 17
    assert lib.fa_paged_num_splits(1, 4, 2, 1, 64, 32, 1) == 1
    assert lib.fa_paged_num_splits(1, 4, 2, 1, 64, 48, 10) == 0
    assert lib.fa_paged_num_splits(1, 4, 2, 1, 96, 32, 10) == 0


def test_paged_form_choice(lib):
    """0 = the prefill form: many query rows per KV head (or d = 96) with
    pages of at least 64 keys and at most 8192 pages per sequence."""
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 64, 64, 10) == 0
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 96, 64, 10) == 0
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 128, 256, 8192) == 0
    # 32-key pages, too many pages, d = 256: the KV-split form
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 64, 32, 10) >= 1
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 64, 64, 8193) >= 1
    assert lib.fa_paged_num_splits(1, 4, 2, 100, 256, 64, 10) >= 1
    # few rows per KV head: the KV-split form
    assert lib.fa_paged_num_splits(1, 4, 2, 32, 64, 64, 10) >= 1


def test_paged_prefill_form_passes_validation(lib):
    """The prefill form takes no workspace; these calls pass every check
    and reach the device query (FA_ERR_HIP without a GPU)."""
    assert _fresh(lambda: _paged(lib, Nq=100, ps=64, ws=None, wsb=0)) == \
        _lib.FA_ERR_HIP
    assert _fresh(lambda: _paged(lib, Nq=100, ps=64, d=96)) == _lib.FA_ERR_HIP
    assert _fresh(lambda: _paged(lib, Nq=100, ps=64, d=32, causal=1, wl=50)) \
        == _lib.FA_ERR_HIP


def _kvlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, sl=P, B=2, Hq=4, Hkv=2, Nq=1, Nk=256,
             d=64, causal=0, wl=-1, wr=-1, scale=0.125, out=0, S=0, ws=P,
             wsb=1 << 20)
    a.update(kw)
    return lib.fa_fwd_kvlen(a["q"], a["k"], a["v"], a["o"], a["lse"],
                            a["sl"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                            a["Nk"], a["d"], a["causal"], a["wl"], a["wr"],
                            a["scale"], a["out"], a["S"], a["ws"], a["wsb"],
                            None)


KVLEN_INVALID = [
    dict(q=None), dict(k=P + 2), dict(v=None), dict(o=P + 4), dict(lse=None),
    dict(sl=None), dict(sl=P + 2), dict(B=0), dict(Hq=3), dict(Nq=0),
    dict(Nk=0), dict(wl=-2), dict(wr=-5), dict(scale=-1.0), dict(out=3),
    dict(S=-1), dict(S=4097), dict(ws=None), dict(ws=P + 8), dict(wsb=0),
]


@pytest.mark.parametrize("kw", KVLEN_INVALID, ids=lambda k: str(k))
def test_kvlen_invalid_arguments(lib, kw):
    assert _kvlen(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_kvlen_unsupported(lib):
    # d = 96 runs only in the prefill form (num_splits = 0)
    assert _kvlen(lib, d=96, S=2) == _lib.FA_ERR_UNSUPPORTED
    assert _kvlen(lib, Nk=1 << 24, d=128) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def test_kvlen_prefill_form_passes_validation(lib):
    """Many query rows per KV head (or d = 96) take the prefill form, with
    no workspace: the calls reach the device query (FA_ERR_HIP here)."""
    assert _fresh(lambda: _kvlen(lib, Nq=100, ws=None, wsb=0)) == \
        _lib.FA_ERR_HIP
    assert _fresh(lambda: _kvlen(lib, d=96)) == _lib.FA_ERR_HIP
    # an explicit split count keeps the KV-split form and its workspace
    assert _kvlen(lib, Nq=100, S=2, ws=None) == _lib.FA_ERR_INVALID_ARG


def _colmask(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cb=P, B=1, Hq=4, Hkv=2, Nq=64, Nk=64,
             d=64, causal=1, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd_colmask(a["q"], a["k"], a["v"], a["o"], a["lse"],
                              a["cb"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                              a["Nk"], a["d"], a["causal"], a["scale"],
                              a["out"], None)


COLMASK_INVALID = [
    dict(q=None), dict(k=P + 2), dict(v=None), dict(o=P + 4), dict(lse=None),
    dict(cb=None), dict(cb=P + 4), dict(B=0), dict(Hq=3), dict(Nq=0),
    dict(Nk=0), dict(scale=-1.0), dict(out=3),
]


@pytest.mark.parametrize("kw", COLMASK_INVALID, ids=lambda k: str(k))
def test_colmask_invalid_arguments(lib, kw):
    assert _colmask(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_colmask_unsupported(lib):
    assert _colmask(lib, d=256) == _lib.FA_ERR_UNSUPPORTED
    assert _fresh(lambda: _colmask(lib, d=96)) == _lib.FA_ERR_HIP
    assert _colmask(lib, Nk=64 * 8192) == _lib.FA_ERR_UNSUPPORTED
    assert _colmask(lib, Nk=64 * 6655 + 1) == _lib.FA_ERR_UNSUPPORTED
    # the largest key count passes validation (no device here)
    assert _fresh(lambda: _colmask(lib, Nk=64 * 6655)) == _lib.FA_ERR_HIP
    assert lib.fa_last_hip_error() == 0


def _fp8(lib, **kw):
    a = dict(q=P, k=P, vt=P, qd=P, kd=P, vd=P, o=P, lse=P, B=1, Hq=4, Hkv=2,
             Nq=16, Nk=16, ldv=64, d=128, causal=0, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd_fp8(a["q"], a["k"], a["vt"], a["qd"], a["kd"], a["vd"],
                          a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Nq"], a["Nk"], a["ldv"], a["d"], a["causal"],
                          a["scale"], a["out"], None)


FP8_INVALID = [
    dict(q=None), dict(k=P + 8), dict(vt=None), dict(o=P + 2), dict(lse=None),
    dict(qd=None), dict(kd=P + 2), dict(vd=None), dict(B=0), dict(Hq=3),
    dict(Nq=0), dict(Nk=0), dict(ldv=8), dict(ldv=65), dict(Nk=65, ldv=64),
    dict(scale=math.nan), dict(out=7),
]


@pytest.mark.parametrize("kw", FP8_INVALID, ids=lambda k: str(k))
def test_fp8_invalid_arguments(lib, kw):
    assert _fp8(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_fp8_unsupported(lib):
    assert _fp8(lib, d=64) == _lib.FA_ERR_UNSUPPORTED
    assert _fp8(lib, d=96) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def _strided(lib, **kw):
    import ctypes
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=64,
             qs=(4096, 1024, 64), ks=(2048, 1024, 64), vs=(2048, 1024, 64),
             os_=(4096, 1024, 64), causal=0, wl=-1, wr=-1, scale=0.125, out=0)
    a.update(kw)
    arr = lambda t: None if t is None else ctypes.addressof((ctypes.c_longlong * 3)(*t))
    keep = [(ctypes.c_longlong * 3)(*t) if t is not None else None
            for t in (a["qs"], a["ks"], a["vs"], a["os_"])]
    ptrs = [ctypes.addressof(x) if x is not None else None for x in keep]
    return lib.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"],
                              a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                              a["d"], *ptrs, a["causal"], a["wl"], a["wr"],
                              a["scale"], a["out"], None)


STRIDED_INVALID = INVALID + [
    dict(qs=None), dict(os_=None), dict(ks=(2048, 1024, 60)),
    dict(vs=(2048, 4, 64)), dict(qs=(-8, 1024, 64)), dict(os_=(4096, 1024, 32)),
    dict(wl=-2),
]


@pytest.mark.parametrize("kw", STRIDED_INVALID, ids=lambda k: str(k))
def test_strided_invalid_arguments(lib, kw):
    assert _strided(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_strided_unsupported(lib):
    assert _strided(lib, d=256, qs=(4096, 1024, 256), ks=(2048, 1024, 256),
                    vs=(2048, 1024, 256), os_=(4096, 1024, 256)) == \
        _lib.FA_ERR_UNSUPPORTED
    assert _fresh(lambda: _strided(
        lib, d=96, qs=(4096, 1024, 96), ks=(2048, 1024, 96),
        vs=(2048, 1024, 96), os_=(4096, 1024, 96))) == _lib.FA_ERR_HIP
    # one K head spans (Nk - 1) * row stride * 2 + 2d bytes
    assert _strided(lib, Nk=(1 << 16) + 2, ks=(0, 0, 1 << 14)) == \
        _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def _sparse(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, m=P, mb=0, mh=0, B=1, Hq=4, Hkv=2,
             Nq=16, Nk=16, d=64, causal=0, scale=0.125, out=0)
    a.update(kw)
    return lib.fa_fwd_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"],
                                   a["m"], a["mb"], a["mh"], a["B"], a["Hq"],
                                   a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                   a["causal"], a["scale"], a["out"], None)


@pytest.mark.parametrize("kw", INVALID + [dict(m=None), dict(mb=-1),
                                          dict(mh=-4)], ids=lambda k: str(k))
def test_sparse_invalid_arguments(lib, kw):
    assert _sparse(lib, **kw) == _lib.FA_ERR_INVALID_ARG


def test_sparse_unsupported(lib):
    assert _sparse(lib, d=256) == _lib.FA_ERR_UNSUPPORTED
    assert _fresh(lambda: _sparse(lib, d=96)) == _lib.FA_ERR_HIP
    assert _sparse(lib, Nk=8191 * 64 + 1) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_hip_error() == 0


def test_library_matches_its_sources(lib):
    """The loaded library reports the hash of the sources on disk, and the
    same digits sit behind the file's marker."""
    from exact_io_aware_05_amd import build
    want = build.source_hash()
    assert lib.fa_source_hash().decode() == want
    assert build.embedded_hash(_lib.LIB_PATH) == want
    assert re.fullmatch(r"[0-9a-f]{64}", want)


def test_source_hash_covers_headers_and_flags(monkeypatch, tmp_path):
    """Editing any kernel source or header, or the flags, changes the hash."""
    from exact_io_aware_05_amd import build
    base = build.source_hash()
    files = build.source_files()
    names = {os.path.basename(f) for f in files}
    assert {"fa_prefill.hip", "fa_device.h", "fa_internal.h", "fa.h"} <= names
    victim = next(f for f in files if f.endswith("fa_device.h"))
    orig_open = open

    def patched_open(path, mode="r", *a, **k):
        if os.path.abspath(path) == victim and "b" in mode:
            data = orig_open(path, mode, *a, **k).read() + b"\n// edit\n"
            p = tmp_path / "edited"
            p.write_bytes(data)
            return orig_open(p, mode, *a, **k)
        return orig_open(path, mode, *a, **k)

    monkeypatch.setattr("builtins.open", patched_open)
    assert build.source_hash() != base
    monkeypatch.undo()
    assert build.source_hash() == base
    monkeypatch.setattr(build, "EXTRA", {**build.EXTRA, "fa_api.hip": ["-O1"]})
    assert build.source_hash() != base


def test_source_hash_does_not_depend_on_the_tree_location(tmp_path):
    """A copy of the sources at another path (as on a remote host) hashes
    the same, so a library built here is not taken for stale there."""
    import shutil
    from exact_io_aware_05_amd import build
    root = tmp_path / "elsewhere"
    shutil.copytree(build.PKG, root / "exact_io_aware_05_amd",
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    shutil.copytree(build.INCLUDE, root / "include")
    code = ("import sys; sys.path.insert(0, sys.argv[1]); "
            "from exact_io_aware_05_amd import build; "
            "print(build.ROOT); print(build.source_hash())")
    out = subprocess.run([sys.executable, "-c", code, str(root)],
                         capture_output=True, text=True, check=True)
    where, digest = out.stdout.split()
    assert os.path.realpath(where) == os.path.realpath(root)
    assert digest == build.source_hash()


def test_stale_library_is_refused_without_a_compiler(monkeypatch, tmp_path):
    """A library whose embedded hash differs from the sources is never
    loaded: with no hipcc to rebuild it, load() raises."""
    import shutil
    from exact_io_aware_05_amd import build
    stale = tmp_path / "libfa.so"
    shutil.copy(_lib.LIB_PATH, stale)
    monkeypatch.setattr(_lib, "LIB_PATH", str(stale))
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 64)

    def no_hipcc():
        raise RuntimeError("hipcc not found")

    monkeypatch.setattr(build, "hipcc", no_hipcc)
    with pytest.raises(_lib.StaleLibraryError):
        _lib.load()
    # a library with no marker at all is stale too
    stale.write_bytes(b"\x7fELF not a library")
    assert build.embedded_hash(str(stale)) is None
    with pytest.raises(_lib.StaleLibraryError):
        _lib.load()


def test_noalloc_scratch_limit(lib):
    """fa_fwd_noalloc refuses, before any HIP call, a KV-split call whose
    partials exceed its fixed scratch array; the limit is reported."""
    cap = lib.fa_noalloc_scratch_bytes()
    assert cap == 16 << 20
    B, Hq, Hkv, Nq, Nk, d = 1024, 32, 8, 1, 32768, 128
    S = lib.fa_default_num_splits(B, Hq, Hkv, Nq, Nk, d)
    assert S >= 1
    need = lib.fa_splitkv_workspace_bytes(B, Hq, Nq, d, S)
    assert need > cap
    st = lib.fa_fwd_noalloc(P, P, P, P, P, B, Hq, Hkv, Nq, Nk, d, 0, 0.088,
                            0, None)
    assert st == _lib.FA_ERR_TOO_LARGE
    assert b"FA_ERR_TOO_LARGE" in lib.fa_status_string(st)
    # invalid arguments are still reported as such
    assert lib.fa_fwd_noalloc(None, P, P, P, P, 1, 4, 2, 1, 64, 64, 0, 0.125,
                              0, None) == _lib.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_noalloc(P, P, P, P, P, 1, 4, 2, 1, 64, 100, 0, 0.125,
                              0, None) == _lib.FA_ERR_UNSUPPORTED
