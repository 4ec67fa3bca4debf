"""Fused exact attention forward and backward for AMD MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind the C
interface of ``include/fa.h``); ``ops`` is its PyTorch binding.
"""
import importlib

from ._lib import FAError, load  # noqa: F401

_LAZY = ("fa_fwd", "fa_fwd_splitkv", "splitkv_workspace_bytes",
         "default_num_splits", "fa_bwd", "bwd_workspace_bytes",
         "fa_fwd_varlen", "fa_fwd_window",
         "fa_fwd_paged", "paged_num_splits", "fa_fwd_fp8", "fa_fwd_strided",
         "fa_fwd_block_sparse", "fa_fwd_kvlen", "fa_fwd_colmask")


def __getattr__(name):
    # the torch binding is imported on first use, so that loading the C
    # library does not require torch
    if name == "ops" or name in _LAZY:
        ops = importlib.import_module(__name__ + ".ops")
        return ops if name == "ops" else getattr(ops, name)
    raise AttributeError(name)
