"""PyTorch-facing binding of the attention library.

Argument marshalling only: tensors supply device pointers, shapes and the
current HIP stream; every step of the computation runs in the HIP kernels of
``libfa.so``.  Layouts (contiguous, head dimension fastest):

    q [B, Hq, Nq, d] bf16,  k, v [B, Hkv, Nk, d] bf16
    o [B, Hq, Nq, d] bf16 or fp32,  lse [B, Hq, Nq] fp32 (natural log)
    backward: do [B, Hq, Nq, d] bf16; dq like q, dk and dv like k, in bf16
    or fp32
"""
from __future__ import annotations

import math

import torch

from ._lib import FA_OUT_BF16, FA_OUT_F32, check, load

__all__ = ["fa_fwd", "fa_fwd_splitkv", "splitkv_workspace_bytes",
           "default_num_splits", "fa_bwd", "bwd_workspace_bytes",
           "fa_fwd_varlen", "fa_fwd_window", "fa_fwd_paged", "fa_fwd_kvlen", "fa_fwd_colmask",
           "paged_num_splits", "fa_fwd_fp8", "fa_fwd_strided",
           "fa_fwd_block_sparse"]


def _dims(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, H, N, d]")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    return B, Hq, Hkv, Nq, Nk, d


def _out(q, B, Hq, Nq, d, out_dtype, o, lse):
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=out_dtype, device=q.device)
    elif (o.dtype != out_dtype or tuple(o.shape) != (B, Hq, Nq, d)
          or not o.is_contiguous()):
        raise ValueError("o has the wrong dtype, shape or layout")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq)
          or not lse.is_contiguous()):
        raise ValueError("lse has the wrong dtype, shape or layout")
    return o, lse


def _stream(q):
    return torch.cuda.current_stream(q.device).cuda_stream


def fa_fwd(q, k, v, causal=False, scale=None, out_dtype=torch.bfloat16,
           o=None, lse=None):
    """Attention forward through ``fa_fwd``; returns ``(o, lse)``."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                       scale,
                       FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16,
                       _stream(q))
    check(st, "fa_fwd")
    return o, lse


def fa_fwd_noalloc(q, k, v, causal=False, scale=None,
                   out_dtype=torch.bfloat16, o=None, lse=None):
    """``fa_fwd`` through ``fa_fwd_noalloc`` (the library allocates no
    device memory; KV-split partials use its fixed scratch array).  Returns
    ``(o, lse)``."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_noalloc")
    return o, lse


def fa_fwd_window(q, k, v, window, causal=False, scale=None,
                  out_dtype=torch.bfloat16, o=None, lse=None):
    """Sliding-window forward through ``fa_fwd_window``; ``window`` is
    ``(left, right)`` keys around each query's place on the key axis, -1
    for no bound on a side.  Returns ``(o, lse)``."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    left, right = (int(x) for x in window)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd_window(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), left, right, scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_window")
    return o, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                  max_seqlen_k, causal=False, scale=None,
                  out_dtype=torch.bfloat16, o=None, lse=None):
    """Packed variable-length forward through ``fa_fwd_varlen``.

    q [total_q, Hq, d], k and v [total_k, Hkv, d] (bf16, contiguous),
    cu_seqlens_q / cu_seqlens_k int32 device tensors of B + 1 row offsets;
    returns ``(o, lse)`` with o [total_q, Hq, d] and lse [Hq, total_q]."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if (not isinstance(t, torch.Tensor) or t.dim() != 3
                or t.dtype != torch.bfloat16 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 device tensor "
                             "[total, H, d]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or t.dim() != 1
                or t.dtype != torch.int32 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 device "
                             "tensor")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need B + 1 entries")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if o is None:
        o = torch.empty((total_q, Hq, d), dtype=out_dtype, device=q.device)
    elif (o.dtype != out_dtype or tuple(o.shape) != (total_q, Hq, d)
          or not o.is_contiguous()):
        raise ValueError("o has the wrong dtype, shape or layout")
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)
          or not lse.is_contiguous()):
        raise ValueError("lse has the wrong dtype, shape or layout")
    st = load().fa_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv,
        total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), d,
        int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_varlen")
    return o, lse


def splitkv_workspace_bytes(B, Hq, Nq, d, num_splits) -> int:
    return int(load().fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits))


def default_num_splits(B, Hq, Hkv, Nq, Nk, d) -> int:
    return int(load().fa_default_num_splits(B, Hq, Hkv, Nq, Nk, d))


def fa_fwd_splitkv(q, k, v, num_splits, causal=False, scale=None,
                   out_dtype=torch.bfloat16, o=None, lse=None, workspace=None):
    """KV-split forward through ``fa_fwd_splitkv`` with a torch-allocated
    workspace (uint8 device tensor); returns ``(o, lse)``."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    need = splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = load().fa_fwd_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16,
        int(num_splits), workspace.data_ptr(), workspace.numel(), _stream(q))
    check(st, "fa_fwd_splitkv")
    return o, lse


def bwd_workspace_bytes(B, Hq, Nq) -> int:
    return int(load().fa_bwd_workspace_bytes(B, Hq, Nq))


def _grad(name, t, shape, dtype, like):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} has the wrong dtype, shape or layout")
    return t


def fa_bwd(q, k, v, o, lse, do, causal=False, scale=None,
           grad_dtype=torch.bfloat16, dq=None, dk=None, dv=None,
           workspace=None, window=None):
    """Attention backward through ``fa_bwd`` from the forward inputs, its
    bf16 output ``o`` and ``lse``, and the incoming gradient ``do``;
    returns ``(dq, dk, dv)``.  With ``window = (left, right)`` it runs
    ``fa_bwd_window`` (the mask of ``fa_fwd_window``)."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    for name, t in (("o", o), ("do", do)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16
                or tuple(t.shape) != (B, Hq, Nq, d) or not t.is_contiguous()
                or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous bf16 device tensor "
                             "shaped like q")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, Nq]")
    if grad_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("grad_dtype must be torch.bfloat16 or torch.float32")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = _grad("dq", dq, q.shape, grad_dtype, q)
    dk = _grad("dk", dk, k.shape, grad_dtype, q)
    dv = _grad("dv", dv, k.shape, grad_dtype, q)
    need = bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    gd = FA_OUT_F32 if grad_dtype == torch.float32 else FA_OUT_BF16
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
            dv.data_ptr())
    if window is None:
        st = load().fa_bwd(*ptrs, B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                           scale, gd, workspace.data_ptr(), workspace.numel(),
                           _stream(q))
        check(st, "fa_bwd")
    else:
        left, right = (int(x) for x in window)
        st = load().fa_bwd_window(*ptrs, B, Hq, Hkv, Nq, Nk, d,
                                  int(bool(causal)), left, right, scale, gd,
                                  workspace.data_ptr(), workspace.numel(),
                                  _stream(q))
        check(st, "fa_bwd_window")
    return dq, dk, dv


def paged_num_splits(B, Hq, Hkv, Nq, d, page_size, max_pages_per_seq) -> int:
    return int(load().fa_paged_num_splits(B, Hq, Hkv, Nq, d, page_size,
                                          max_pages_per_seq))


def fa_fwd_paged(q, k_cache, v_cache, page_table, seqlens_k, causal=False,
                 scale=None, window=(-1, -1), out_dtype=torch.bfloat16,
                 num_splits=0, o=None, lse=None, workspace=None):
    """Forward over a paged KV cache through ``fa_fwd_paged``.

    q [B, Hq, Nq, d] bf16; k_cache, v_cache [num_pages, page_size, Hkv, d]
    bf16; page_table int32 [B, max_pages_per_seq] and seqlens_k int32 [B]
    on the device.  Returns ``(o, lse)`` shaped like ``fa_fwd``'s."""
    if (not isinstance(q, torch.Tensor) or q.dim() != 4
            or q.dtype != torch.bfloat16 or not q.is_cuda
            or not q.is_contiguous()):
        raise ValueError("q must be a contiguous bf16 device tensor "
                         "[B, Hq, Nq, d]")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if (not isinstance(t, torch.Tensor) or t.dim() != 4
                or t.dtype != torch.bfloat16 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 device tensor "
                             "[num_pages, page_size, Hkv, d]")
    if tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("k_cache and v_cache differ in shape")
    B, Hq, Nq, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head dimensions differ")
    for name, t, shape in (("page_table", page_table, None),
                           ("seqlens_k", seqlens_k, (B,))):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32
                or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages_per_seq]")
    if tuple(seqlens_k.shape) != (B,):
        raise ValueError("seqlens_k must be [B]")
    max_pages = page_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    # (0: the library runs the prefill form, which takes no workspace)
    splits = int(num_splits) or paged_num_splits(B, Hq, Hkv, Nq, d, page_size,
                                                 max_pages)
    if workspace is None:
        need = splitkv_workspace_bytes(B, Hq, Nq, d, splits) if splits else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8,
                                device=q.device)
    left, right = (int(x) for x in window)
    st = load().fa_fwd_paged(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
        lse.data_ptr(), page_table.data_ptr(), seqlens_k.data_ptr(), B, Hq,
        Hkv, Nq, d, num_pages, page_size, max_pages, int(bool(causal)), left,
        right, scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, splits,
        workspace.data_ptr(), workspace.numel(), _stream(q))
    check(st, "fa_fwd_paged")
    return o, lse


def fa_fwd_colmask(q, k, v, col_bounds, causal=False, scale=None,
                   out_dtype=torch.bfloat16, o=None, lse=None):
    """Forward with a column-interval mask through ``fa_fwd_colmask``.

    col_bounds int32 [B, Nk, 2] on the device: key j of sequence b may be
    seen by query rows col_bounds[b, j, 0] .. col_bounds[b, j, 1] - 1.
    Returns ``(o, lse)`` shaped like ``fa_fwd``'s."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    if (not isinstance(col_bounds, torch.Tensor)
            or col_bounds.dtype != torch.int32 or not col_bounds.is_cuda
            or not col_bounds.is_contiguous()
            or tuple(col_bounds.shape) != (B, Nk, 2)):
        raise ValueError("col_bounds must be a contiguous int32 device "
                         "tensor [B, Nk, 2]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd_colmask(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        lse.data_ptr(), col_bounds.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
        int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_colmask")
    return o, lse


def fa_fwd_kvlen(q, k, v, seqlens_k, causal=False, scale=None,
                 window=(-1, -1), out_dtype=torch.bfloat16, num_splits=0,
                 o=None, lse=None, workspace=None):
    """Variable-length decode over a padded cache through ``fa_fwd_kvlen``.

    q [B, Hq, Nq, d] bf16; k, v [B, Hkv, Nk, d] bf16 padded to the longest
    sequence; seqlens_k int32 [B] on the device (sequence b uses its first
    seqlens_k[b] rows).  Returns ``(o, lse)`` shaped like ``fa_fwd``'s."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    if (not isinstance(seqlens_k, torch.Tensor)
            or seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda
            or not seqlens_k.is_contiguous()
            or tuple(seqlens_k.shape) != (B,)):
        raise ValueError("seqlens_k must be a contiguous int32 device "
                         "tensor [B]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    # (0: the library runs the prefill form, which takes no workspace)
    splits = int(num_splits) or default_num_splits(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None:
        need = splitkv_workspace_bytes(B, Hq, Nq, d, splits) if splits else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8,
                                device=q.device)
    left, right = (int(x) for x in window)
    st = load().fa_fwd_kvlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        lse.data_ptr(), seqlens_k.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
        int(bool(causal)), left, right, scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, splits,
        workspace.data_ptr(), workspace.numel(), _stream(q))
    check(st, "fa_fwd_kvlen")
    return o, lse


def fa_fwd_fp8(q8, k8, vt8, q_descale, k_descale, v_descale, causal=False,
               scale=None, out_dtype=torch.bfloat16, o=None, lse=None):
    """FP8 (E4M3) forward through ``fa_fwd_fp8``.

    q8 [B, Hq, Nq, d], k8 [B, Hkv, Nk, d] and vt8 [B, Hkv, d, ldv] (V
    transposed, ldv >= Nk a multiple of 64) are uint8 device tensors of
    E4M3 codes; the descales are fp32 device tensors [B, Hq], [B, Hkv],
    [B, Hkv].  Returns ``(o, lse)`` shaped like ``fa_fwd``'s."""
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        if (not isinstance(t, torch.Tensor) or t.dim() != 4
                or t.dtype != torch.uint8 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous uint8 device "
                             "tensor of E4M3 codes")
    B, Hq, Nq, d = q8.shape
    Bk, Hkv, Nk, dk = k8.shape
    if Bk != B or dk != d or tuple(vt8.shape[:3]) != (B, Hkv, d):
        raise ValueError("shape mismatch between q8, k8 and vt8")
    ldv = vt8.shape[3]
    for name, t, shape in (("q_descale", q_descale, (B, Hq)),
                           ("k_descale", k_descale, (B, Hkv)),
                           ("v_descale", v_descale, (B, Hkv))):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32
                or not t.is_cuda or not t.is_contiguous()
                or tuple(t.shape) != shape):
            raise ValueError(f"{name} must be a contiguous fp32 device "
                             f"tensor {shape}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q8, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd_fp8(
        q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), q_descale.data_ptr(),
        k_descale.data_ptr(), v_descale.data_ptr(), o.data_ptr(),
        lse.data_ptr(), B, Hq, Hkv, Nq, Nk, ldv, d, int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q8))
    check(st, "fa_fwd_fp8")
    return o, lse


def fa_fwd_strided(q, k, v, causal=False, scale=None, window=(-1, -1),
                   out_dtype=torch.bfloat16, o=None, lse=None):
    """Forward through ``fa_fwd_strided`` on 4-D bf16 views indexed
    [B, H, N, d] (any strides, head dimension contiguous, strides multiples
    of 8); ``o`` may be a strided view too (default: a new contiguous
    tensor).  Returns ``(o, lse)``."""
    import ctypes
    for name, t in (("q", q), ("k", k), ("v", v)):
        if (not isinstance(t, torch.Tensor) or t.dim() != 4
                or t.dtype != torch.bfloat16 or not t.is_cuda
                or t.stride(3) != 1):
            raise ValueError(f"{name} must be a bf16 device tensor viewed as "
                             "[B, H, N, d] with the head dimension contiguous")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=out_dtype, device=q.device)
    elif (o.dtype != out_dtype or tuple(o.shape) != (B, Hq, Nq, d)
          or o.stride(3) != 1):
        raise ValueError("o has the wrong dtype, shape or layout")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq)
          or not lse.is_contiguous()):
        raise ValueError("lse has the wrong dtype, shape or layout")
    arr = lambda t: (ctypes.c_longlong * 3)(t.stride(0), t.stride(1),
                                            t.stride(2))
    qs, ks, vs, os_ = arr(q), arr(k), arr(v), arr(o)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    left, right = (int(x) for x in window)
    st = load().fa_fwd_strided(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, ctypes.addressof(qs),
        ctypes.addressof(ks), ctypes.addressof(vs), ctypes.addressof(os_),
        int(bool(causal)), left, right, scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_strided")
    return o, lse


SPARSE_BLOCK = (128, 64)  # query rows, keys per block of a block mask


def fa_fwd_block_sparse(q, k, v, block_mask, causal=False, scale=None,
                        out_dtype=torch.bfloat16, o=None, lse=None):
    """Block-sparse forward through ``fa_fwd_block_sparse``.

    block_mask: uint8 device tensor [Bm, Hm, ceil(Nq / 128), ceil(Nk / 64)]
    with Bm in (1, B) and Hm in (1, Hq) (size-1 axes are shared), its last
    two axes contiguous.  Returns ``(o, lse)`` like ``fa_fwd``."""
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    nqb = (Nq + SPARSE_BLOCK[0] - 1) // SPARSE_BLOCK[0]
    nkb = (Nk + SPARSE_BLOCK[1] - 1) // SPARSE_BLOCK[1]
    m = block_mask
    if (not isinstance(m, torch.Tensor) or m.dtype != torch.uint8
            or not m.is_cuda or m.dim() != 4 or tuple(m.shape[2:]) != (nqb, nkb)
            or m.shape[0] not in (1, B) or m.shape[1] not in (1, Hq)
            or m.stride(3) != 1 or m.stride(2) != nkb):
        raise ValueError(f"block_mask must be a uint8 device tensor "
                         f"[1 or B, 1 or Hq, {nqb}, {nkb}], rows contiguous")
    mb = m.stride(0) if m.shape[0] == B and B > 1 else 0
    mh = m.stride(1) if m.shape[1] == Hq and Hq > 1 else 0
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _out(q, B, Hq, Nq, d, out_dtype, o, lse)
    st = load().fa_fwd_block_sparse(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        m.data_ptr(), mb, mh, B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
        FA_OUT_F32 if out_dtype == torch.float32 else FA_OUT_BF16, _stream(q))
    check(st, "fa_fwd_block_sparse")
    return o, lse
