"""ctypes loader for ``libfa.so`` (the C interface declared in include/fa.h).

The library is the only compute path: if it is missing it is built from
source with hipcc, and if it cannot be loaded an error is raised.  There is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_ERR_TOO_LARGE = 4
FA_OUT_BF16, FA_OUT_F32 = 0, 1

_c_int, _c_float, _c_size, _vp = (ctypes.c_int, ctypes.c_float,
                                  ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes), mirroring include/fa.h
SIGNATURES = {
    "fa_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                        _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp]),
    "fa_fwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_float, _c_int, _vp]),
    "fa_noalloc_scratch_bytes": (_c_size, []),
    "fa_splitkv_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int,
                                             _c_int]),
    "fa_fwd_splitkv": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_float, _c_int, _c_int, _vp, _c_size, _vp]),
    "fa_default_num_splits": (_c_int, [_c_int] * 6),
    "fa_fwd_window": (_c_int, [_vp] * 5 + [_c_int] * 9 + [_c_float, _c_int,
                                                           _vp]),
    "fa_paged_num_splits": (_c_int, [_c_int] * 7),
    "fa_fwd_colmask": (_c_int, [_vp] * 6 + [_c_int] * 7 + [_c_float, _c_int,
                                                        _vp]),
    "fa_fwd_kvlen": (_c_int, [_vp] * 6 + [_c_int] * 9 + [_c_float, _c_int,
                                                      _c_int, _vp, _c_size,
                                                      _vp]),
    "fa_fwd_paged": (_c_int, [_vp] * 7 + [_c_int] * 11 + [_c_float, _c_int,
                                                           _c_int, _vp,
                                                           _c_size, _vp]),
    "fa_fwd_fp8": (_c_int, [_vp] * 8 + [_c_int] * 8 + [_c_float, _c_int,
                                                       _vp]),
    "fa_fwd_strided": (_c_int, [_vp] * 5 + [_c_int] * 6 + [_vp] * 4 +
                       [_c_int] * 3 + [_c_float, _c_int, _vp]),
    "fa_fwd_block_sparse": (_c_int, [_vp] * 6 + [ctypes.c_longlong] * 2 +
                            [_c_int] * 7 + [_c_float, _c_int, _vp]),
    "fa_fwd_varlen": (_c_int, [_vp] * 7 + [_c_int] * 9 + [_c_float, _c_int,
                                                           _vp]),
    "fa_bwd_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "fa_bwd": (_c_int, [_vp] * 9 + [_c_int] * 7 + [_c_float, _c_int, _vp,
                                                   _c_size, _vp]),
    "fa_bwd_window": (_c_int, [_vp] * 9 + [_c_int] * 9 + [_c_float, _c_int,
                                                           _vp, _c_size, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
    "fa_last_hip_error": (_c_int, []),
    "fa_source_hash": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.fa_status_string(status).decode()
        if status == FA_ERR_HIP:
            msg += f" (hipError_t {lib.fa_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


class StaleLibraryError(RuntimeError):
    """libfa.so was built from other sources than the ones beside it."""


def _fresh_or_rebuild():
    """Make sure libfa.so exists and was built from the sources on disk:
    build it when it is missing or stale and hipcc is available, otherwise
    raise StaleLibraryError.  Returns the expected source hash."""
    from . import build as _build
    want = _build.source_hash()
    have = _build.embedded_hash(LIB_PATH)
    if have == want:
        return want
    try:
        _build.hipcc()
    except RuntimeError:
        raise StaleLibraryError(
            f"{LIB_PATH} was built from other sources (library {have}, "
            f"sources {want}) and hipcc is not available to rebuild it")
    _build.build()
    if _build.embedded_hash(LIB_PATH) != want:
        raise StaleLibraryError(f"rebuilt {LIB_PATH} does not match its sources")
    return want


def load():
    """Load libfa.so, building it first if it is missing or was built from
    other sources than the ones on disk (see ``fa_source_hash``)."""
    global _lib
    with _lock:
        if _lib is None:
            want = _fresh_or_rebuild()
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            got = lib.fa_source_hash().decode()
            if got != want:
                raise StaleLibraryError(
                    f"loaded {LIB_PATH} reports source hash {got}, "
                    f"sources hash to {want}")
            _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FAError(status, where)
