"""Python binding of libfa.so, the gfx950 exact tiled attention library.

Argument marshalling only: every step of the attention computation runs in
the HIP kernels behind the C ABI declared in ``include/fa.h``. PyTorch
supplies device memory and the current stream; nothing here computes.

Low-level calls mirror the C ABI names (``fa_fwd``, ``fa_bwd``,
``fa_bwd_workspace_bytes``, ``fa_status_string``, ``fa_fwd_varlen``,
``fa_bwd_varlen``, ``fa_bwd_varlen_workspace_bytes``) and take raw integer
device pointers. ``forward`` / ``backward`` are conveniences that take torch
tensors of shape [B, H, N, d] and allocate the outputs; ``forward_varlen`` /
``backward_varlen`` take packed [tokens, heads, d] tensors with cumulative
sequence offsets.

There is no fallback: if ``libfa.so`` has not been built, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch  # loads the HIP runtime first, so libfa.so binds to the same one

__all__ = [
    "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_MASK",
    "FA_ERR_WORKSPACE", "FA_ERR_ALIGN", "FA_ERR_HIP", "FA_ERR_ARG", "FA_ERR_SCRATCH", "FA_BWD_NOALLOC_MAX_ROWS",
    "MASK_NONE", "MASK_CAUSAL", "MASK_BLOCK_SPARSE", "DTYPE_BF16", "DTYPE_F32",
    "FAError", "fa_fwd", "fa_fwd_tiled", "fa_bwd", "fa_bwd_rowterm", "fa_bwd_dkdv", "fa_bwd_dq",
    "fa_bwd_workspace_bytes", "fa_status_string", "fa_fwd_varlen", "fa_bwd_varlen",
    "fa_bwd_varlen_workspace_bytes", "fa_splitkv_splits", "fa_splitkv_workspace_bytes", "fa_fwd_splitkv",
    "fa_fwd_fp8", "fa_bwd_noalloc", "fa_debug_reverse_order", "forward", "backward", "backward_noalloc", "forward_varlen", "backward_varlen", "forward_splitkv", "forward_fp8",
    "library_path", "lib",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, -1, -2, -3
FA_ERR_MASK, FA_ERR_WORKSPACE, FA_ERR_ALIGN, FA_ERR_HIP, FA_ERR_ARG, FA_ERR_SCRATCH = -4, -5, -6, -7, -8, -9
FA_BWD_NOALLOC_MAX_ROWS = 1 << 21   # B * H * N limit of fa_bwd_noalloc (its built-in scratch)
MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE = 0, 1, 2
DTYPE_BF16, DTYPE_F32 = 0, 1
MASK_BLOCK = 128

_lib = None


class FAError(RuntimeError):
    """A libfa call returned a negative status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {fa_status_string(status)} (status {status})")


def library_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (loaded on first use; raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m io_aware_exact_10_amd.build` "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
        L.fa_fwd.restype = i
        L.fa_fwd_tiled.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, i, vp]
        L.fa_fwd_tiled.restype = i
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
        L.fa_bwd.restype = i
        L.fa_bwd_rowterm.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.fa_bwd_rowterm.restype = i
        L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
        L.fa_bwd_dkdv.restype = i
        L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
        L.fa_bwd_dq.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp] + [i] * 8 + [f, i, i, vp]
        L.fa_fwd_varlen.restype = i
        L.fa_bwd_varlen.argtypes = [vp] * 11 + [i] * 8 + [f, i, i, vp, sz, vp]
        L.fa_bwd_varlen.restype = i
        L.fa_bwd_varlen_workspace_bytes.argtypes = [i, i, i]
        L.fa_bwd_varlen_workspace_bytes.restype = sz
        L.fa_splitkv_splits.argtypes = [i, i, i, i]
        L.fa_splitkv_splits.restype = i
        L.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i]
        L.fa_splitkv_workspace_bytes.restype = sz
        L.fa_fwd_splitkv.argtypes = [vp] * 7 + [i] * 8 + [f, i, i, i, vp, sz, vp]
        L.fa_fwd_splitkv.restype = i
        L.fa_fwd_fp8.argtypes = [vp] * 5 + [i] * 5 + [f, f, f, f, i, vp]
        L.fa_fwd_fp8.restype = i
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
        L.fa_bwd_noalloc.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_debug_reverse_order.argtypes = [i]
        L.fa_debug_reverse_order.restype = i
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/fa.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", txt)))


# ---------------------------------------------------------------------------
# C ABI mirrors (raw pointers as Python ints)
# ---------------------------------------------------------------------------
def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_debug_reverse_order(on: int) -> int:
    """Debug switch: later launches take their work items in reverse order
    (results must not change). Returns the previous setting."""
    return int(lib().fa_debug_reverse_order(int(on)))


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d))


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask_kind, block_mask, dtype, stream) -> int:
    return int(lib().fa_fwd(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), mask_kind,
                            block_mask, dtype, stream))


def fa_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, mask_kind, block_mask, dtype, block_rows, stream) -> int:
    return int(lib().fa_fwd_tiled(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), mask_kind,
                                  block_mask, dtype, block_rows, stream))


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, mask_kind, block_mask, dtype,
           workspace, workspace_bytes, stream) -> int:
    return int(lib().fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, ctypes.c_float(scale),
                            mask_kind, block_mask, dtype, workspace, workspace_bytes, stream))


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, mask_kind, block_mask, dtype,
                   stream) -> int:
    return int(lib().fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, ctypes.c_float(scale),
                                    mask_kind, block_mask, dtype, stream))


def fa_bwd_rowterm(o, dO, lse, B, H, N, d, dtype, workspace, workspace_bytes, stream) -> int:
    return int(lib().fa_bwd_rowterm(o, dO, lse, B, H, N, d, dtype, workspace, workspace_bytes, stream))


def fa_bwd_dkdv(q, k, v, lse, dO, dk, dv, B, H, N, d, scale, mask_kind, block_mask, dtype,
                workspace, workspace_bytes, stream) -> int:
    return int(lib().fa_bwd_dkdv(q, k, v, lse, dO, dk, dv, B, H, N, d, ctypes.c_float(scale), mask_kind,
                                 block_mask, dtype, workspace, workspace_bytes, stream))


def fa_bwd_dq(q, k, v, lse, dO, dq, B, H, N, d, scale, mask_kind, block_mask, dtype,
              workspace, workspace_bytes, stream) -> int:
    return int(lib().fa_bwd_dq(q, k, v, lse, dO, dq, B, H, N, d, ctypes.c_float(scale), mask_kind,
                               block_mask, dtype, workspace, workspace_bytes, stream))


def fa_bwd_varlen_workspace_bytes(total_q: int, H: int, d: int) -> int:
    return int(lib().fa_bwd_varlen_workspace_bytes(total_q, H, d))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q, max_seqlen_k,
                  total_q, total_k, d, scale, mask_kind, dtype, stream) -> int:
    return int(lib().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q,
                                   max_seqlen_k, total_q, total_k, d, ctypes.c_float(scale), mask_kind,
                                   dtype, stream))


def fa_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q,
                  max_seqlen_k, total_q, total_k, d, scale, mask_kind, dtype, workspace, workspace_bytes,
                  stream) -> int:
    return int(lib().fa_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, H, Hkv,
                                   max_seqlen_q, max_seqlen_k, total_q, total_k, d, ctypes.c_float(scale),
                                   mask_kind, dtype, workspace, workspace_bytes, stream))


def fa_splitkv_splits(B: int, Hkv: int, max_seqlen_k: int, num_splits: int) -> int:
    return int(lib().fa_splitkv_splits(B, Hkv, max_seqlen_k, num_splits))


def fa_splitkv_workspace_bytes(total_q: int, H: int, d: int, splits: int) -> int:
    return int(lib().fa_splitkv_workspace_bytes(total_q, H, d, splits))


def fa_fwd_splitkv(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q, max_seqlen_k,
                   total_q, total_k, d, scale, mask_kind, dtype, num_splits, workspace, workspace_bytes,
                   stream) -> int:
    return int(lib().fa_fwd_splitkv(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q,
                                    max_seqlen_k, total_q, total_k, d, ctypes.c_float(scale), mask_kind, dtype,
                                    num_splits, workspace, workspace_bytes, stream))


def fa_fwd_fp8(q, k, v_t, o, lse, B, H, N, d, ldv, scale, q_descale, k_descale, v_descale, mask_kind,
               stream) -> int:
    return int(lib().fa_fwd_fp8(q, k, v_t, o, lse, B, H, N, d, ldv, ctypes.c_float(scale),
                                ctypes.c_float(q_descale), ctypes.c_float(k_descale), ctypes.c_float(v_descale),
                                mask_kind, stream))


# ---------------------------------------------------------------------------
# torch conveniences
# ---------------------------------------------------------------------------
_DT = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}


def _need(t, name, shape, dtype):
    """Structure of one tensor argument (shape, dtype, contiguity); the
    device is checked separately (``_on_gpu``) after every structural check,
    so a wrong shape is reported whatever device the tensors are on."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_workspace(t, need):
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError("workspace must be a contiguous torch tensor")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes, got {t.numel() * t.element_size()}")


def _on_gpu(device, **tensors):
    """Every tensor argument lives on the GPU that holds q (the kernels take
    raw pointers, so a tensor elsewhere would be read or written out of its
    allocation)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: tensors must be on the GPU")
        if t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_qkv(q, k, v):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")


def _mask_ptr(mask_kind, block_mask, N, device):
    if mask_kind != MASK_BLOCK_SPARSE:
        return None
    if block_mask is None:
        raise ValueError("block_mask is required for MASK_BLOCK_SPARSE")
    nb = -(-N // MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be uint8 [{nb}, {nb}]")
    if not block_mask.is_cuda or not block_mask.is_contiguous() or block_mask.device != device:
        raise ValueError("block_mask must be a contiguous tensor on the same GPU")
    return block_mask.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, scale=None, mask_kind=MASK_NONE, block_mask=None, out=None, lse=None, block_rows=0):
    """Attention forward on the current stream; returns (o, lse).

    q, k, v: contiguous [B, H, N, d] bf16 or fp32 GPU tensors; scale defaults
    to 1/sqrt(d). lse is fp32 [B, H, N] (natural log). ``block_rows`` other
    than 0 (32, 64, 128, 256; bf16) fixes the query rows per workgroup and
    calls fa_fwd_tiled.
    """
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is not None:
        _need(out, "out", q.shape, q.dtype)
    if lse is not None:
        _need(lse, "lse", (B, H, N), torch.float32)
    _on_gpu(q.device, q=q, k=k, v=v, out=out, lse=lse)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    mp = _mask_ptr(mask_kind, block_mask, N, q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            B, H, N, d, scale, mask_kind, mp, _DT[q.dtype])
    if block_rows:
        st, name = fa_fwd_tiled(*args, int(block_rows), _stream(q.device)), "fa_fwd_tiled"
    else:
        st, name = fa_fwd(*args, _stream(q.device)), "fa_fwd"
    if st != FA_OK:
        raise FAError(st, name)
    return o, lse


def backward(q, k, v, o, lse, do, scale=None, mask_kind=MASK_NONE, block_mask=None,
             workspace=None, dq=None, dk=None, dv=None, steps="all"):
    """Attention backward on the current stream; returns (dq, dk, dv).

    ``steps`` selects what is enqueued: "all" (fa_bwd), or one of "rowterm",
    "dkdv", "dq" (the three steps of fa_bwd, for callers that time or
    schedule them separately; "dkdv" and "dq" need the workspace a previous
    "rowterm" call filled).
    """
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    _need(o, "o", q.shape, q.dtype)
    _need(do, "do", q.shape, q.dtype)
    _need(lse, "lse", (B, H, N), torch.float32)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _need(t, name, q.shape, q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is not None:
        _need_workspace(workspace, need)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    mp = _mask_ptr(mask_kind, block_mask, N, q.device)
    wsb = workspace.numel() * workspace.element_size()
    dt = _DT[q.dtype]
    stream = _stream(q.device)
    if steps == "all":
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, mask_kind, mp,
                    dt, workspace.data_ptr(), wsb, stream)
    elif steps == "rowterm":
        st = fa_bwd_rowterm(o.data_ptr(), do.data_ptr(), lse.data_ptr(), B, H, N, d, dt, workspace.data_ptr(), wsb,
                            stream)
    elif steps == "dkdv":
        st = fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                         dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, mask_kind, mp, dt,
                         workspace.data_ptr(), wsb, stream)
    elif steps == "dq":
        st = fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), B, H, N, d, scale, mask_kind, mp, dt, workspace.data_ptr(), wsb, stream)
    else:
        raise ValueError(f"unknown steps {steps!r}")
    if st != FA_OK:
        raise FAError(st, f"fa_bwd ({steps})")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, do, scale=None, mask_kind=MASK_NONE, block_mask=None, dq=None, dk=None,
                     dv=None):
    """``backward`` through fa_bwd_noalloc: no workspace (the library's
    built-in per-GPU scratch holds the row statistics), so with dq, dk, dv
    passed in nothing is allocated. B * H * N <= FA_BWD_NOALLOC_MAX_ROWS."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    _need(o, "o", q.shape, q.dtype)
    _need(do, "do", q.shape, q.dtype)
    _need(lse, "lse", (B, H, N), torch.float32)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _need(t, name, q.shape, q.dtype)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    mp = _mask_ptr(mask_kind, block_mask, N, q.device)
    st = fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, mask_kind, mp,
                        _DT[q.dtype], _stream(q.device))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def _check_varlen(q, k, v, cu_q, cu_k):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [total_q, H, d]; k and v [total_k, Hkv, d]")
    if k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("k and v must match, and share d with q")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name}: q, k, v must be contiguous bfloat16 tensors")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 tensors")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                   mask_kind=MASK_NONE, out=None, lse=None):
    """Packed-batch forward on the current stream; returns (o, lse).

    q: [total_q, H, d]; k, v: [total_k, Hkv, d] (bf16, H a multiple of Hkv);
    cu_seqlens_*: int32 [B + 1] device offsets; lse: fp32 [H, total_q].
    Causal attention aligns each sequence's last query with its last key.
    """
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[:2]
    B = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is not None:
        _need(out, "out", q.shape, q.dtype)
    if lse is not None:
        _need(lse, "lse", (H, Tq), torch.float32)
    _on_gpu(q.device, q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, out=out, lse=lse)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    st = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hkv, int(max_seqlen_q),
                       int(max_seqlen_k), Tq, Tk, d, scale, mask_kind, DTYPE_BF16, _stream(q.device))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_varlen")
    return o, lse


def backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    scale=None, mask_kind=MASK_NONE, workspace=None, dq=None, dk=None, dv=None):
    """Packed-batch backward on the current stream; returns (dq, dk, dv)."""
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[:2]
    B = cu_seqlens_q.numel() - 1
    _need(o, "o", q.shape, q.dtype)
    _need(do, "do", q.shape, q.dtype)
    _need(lse, "lse", (H, Tq), torch.float32)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _need(t, name, ref.shape, ref.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = fa_bwd_varlen_workspace_bytes(Tq, H, d)
    if workspace is not None:
        _need_workspace(workspace, need)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, do=do, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
            dq=dq, dk=dk, dv=dv, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
                       cu_seqlens_k.data_ptr(), B, H, Hkv, int(max_seqlen_q), int(max_seqlen_k), Tq, Tk, d,
                       scale, mask_kind, DTYPE_BF16, workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_varlen")
    return dq, dk, dv


def forward_splitkv(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                    mask_kind=MASK_NONE, num_splits=0, out=None, lse=None, workspace=None):
    """Split-key packed-batch forward (few queries per sequence, long keys);
    same arguments and results as ``forward_varlen``. ``num_splits`` = 0 lets
    the library choose the number of key ranges per sequence."""
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[:2]
    B = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    splits = fa_splitkv_splits(B, Hkv, int(max_seqlen_k), int(num_splits))
    if splits < 0:
        raise FAError(splits, "fa_splitkv_splits")
    need = fa_splitkv_workspace_bytes(Tq, H, d, splits)
    if out is not None:
        _need(out, "out", q.shape, q.dtype)
    if lse is not None:
        _need(lse, "lse", (H, Tq), torch.float32)
    if workspace is not None:
        _need_workspace(workspace, need)
    _on_gpu(q.device, q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, out=out, lse=lse,
            workspace=workspace)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hkv, int(max_seqlen_q),
                        int(max_seqlen_k), Tq, Tk, d, scale, mask_kind, DTYPE_BF16, int(num_splits),
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv")
    return o, lse


def forward_fp8(q, k, v_t, q_descale=1.0, k_descale=1.0, v_descale=1.0, scale=None, mask_kind=MASK_NONE,
                out=None, lse=None):
    """FP8 (E4M3) forward on the current stream; returns (o bf16, lse fp32).

    q, k: uint8 [B, H, N, d] E4M3 codes; v_t: uint8 [B, H, d, ldv], V
    transposed (ldv >= N, a multiple of 16). scale defaults to 1/sqrt(d).
    """
    for t in (q, k, v_t):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v_t must be contiguous uint8 (E4M3 code) tensors of rank 4")
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    B, H, N, d = q.shape
    if tuple(v_t.shape[:3]) != (B, H, d):
        raise ValueError("v_t must be [B, H, d, ldv]")
    ldv = v_t.shape[3]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is not None:
        _need(out, "out", (B, H, N, d), torch.bfloat16)
    if lse is not None:
        _need(lse, "lse", (B, H, N), torch.float32)
    _on_gpu(q.device, q=q, k=k, v_t=v_t, out=out, lse=lse)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v_t.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, ldv,
                    scale, float(q_descale), float(k_descale), float(v_descale), mask_kind, _stream(q.device))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, lse
