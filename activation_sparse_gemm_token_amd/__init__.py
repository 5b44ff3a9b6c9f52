"""Python binding of librtlynx, the MI355X (gfx950) online 2:4
activation-sparse linear layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
of ``librtlynx.so``; PyTorch supplies device memory and the current stream of
the inputs' device (made current for the call).
There is no fallback: if the library is missing or the device is not gfx950
the calls raise.

Entry points (same names as the C ABI in include/rtlynx.h, without the
``rtl_`` prefix):

* ``sparsify_2of4(x, fold_scale=False)`` -> (vals, idx, scale)
* ``sparse_linear(x, w, lora_a=None, lora_b=None, lora_scale=1.0)`` -> y
* ``prepare(x, lora_a=None, lora_scale=1.0)`` -> Prepared, ``apply(prepared, w, lora_b=None)`` -> y
  (the two halves of sparse_linear)
* ``sparse_linear_noalloc(x, w, lora_a=None, lora_b=None, lora_scale=1.0, out=None)`` -> y
  (no workspace: the library's fixed per-GPU scratch array)
* ``dense_linear(x, w)`` -> y
* ``sparse_linear_workspace_bytes(M, K, r)``
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "RtlError", "lib", "library_path", "sparsify_2of4", "sparse_linear", "dense_linear",
    "sparse_linear_workspace_bytes", "version", "status_string", "STATUS", "prepare", "apply", "Prepared",
    "FOLD_SCALE", "MAX_LORA_RANK", "sparse_linear_compressed", "sparse_linear_noalloc", "NOALLOC_SCRATCH_BYTES",
    "COMP_TOKEN", "COMP_NONE", "COMP_TENSOR", "COMP_GROUP", "LORA_RESIDUAL", "LORA_PRUNED", "LORA_INPUT",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librtlynx.so")

STATUS = {
    0: "RTL_OK", 1: "RTL_ERR_NULL_POINTER", 2: "RTL_ERR_BAD_SHAPE", 3: "RTL_ERR_MISALIGNED",
    4: "RTL_ERR_WORKSPACE", 5: "RTL_ERR_NO_DEVICE", 6: "RTL_ERR_UNSUPPORTED_ARCH",
    7: "RTL_ERR_HIP", 8: "RTL_ERR_BAD_FLAGS", 9: "RTL_ERR_STREAM_DEVICE",
}
FOLD_SCALE = 0x1
MAX_LORA_RANK = 128
NOALLOC_SCRATCH_BYTES = 64 << 20
# Variants of the layer (rtl_sparse_linear_prepare_variant): compensation ...
COMP_TOKEN, COMP_NONE, COMP_TENSOR, COMP_GROUP = 0x0, 0x1, 0x2, 0x3
# ... | LoRA input.
LORA_RESIDUAL, LORA_PRUNED, LORA_INPUT = 0x0, 0x4, 0x8

_c_i64, _c_u32, _c_vp, _c_f = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float

_SIGNATURES = {
    "rtl_sparsify_2of4": (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_u32, _c_vp]),
    "rtl_sparse_linear_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "rtl_sparse_linear": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                         _c_f, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "rtl_sparse_linear_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                                 _c_f, _c_vp, _c_vp]),
    "rtl_sparse_linear_prepare": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_f, _c_vp,
                                                 ctypes.c_size_t, _c_vp]),
    "rtl_sparse_linear_apply": (ctypes.c_int, [_c_vp, ctypes.c_size_t, _c_vp, _c_vp, _c_i64, _c_i64,
                                               _c_i64, _c_i64, _c_vp, _c_vp]),
    "rtl_sparse_linear_prepare_variant": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_float,
                                                         _c_u32, _c_vp, ctypes.c_size_t, _c_vp]),
    "rtl_sparse_linear_compressed": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                                    _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "rtl_dense_linear": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "rtl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rtl_version": (ctypes.c_int, []),
}

_lib = None


class RtlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded librtlynx (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"librtlynx.so is not built ({library_path}); run "
                               "python -m activation_sparse_gemm_token_amd.build")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().rtl_status_string(int(status)).decode()


def version() -> int:
    return lib().rtl_version()


def sparse_linear_workspace_bytes(m: int, k: int, r: int) -> int:
    return int(lib().rtl_sparse_linear_workspace_bytes(m, k, r))


def _check(status: int, where: str) -> None:
    if status != 0:
        raise RtlError(status, where)


def _torch():
    import torch
    return torch


def _as_2d(t, name: str):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.reshape(-1, t.shape[-1]) if t.dim() != 2 else t


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _on(device, **tensors):
    """Context in which a call runs: every named tensor on ``device`` (the
    kernels run on one device), which is made current, so that the current
    stream and the library's device are the tensors'."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    return _torch().cuda.device(device)


def _out(out, m: int, n: int, lead, device):
    """A caller's output tensor, or a new one: the kernels write m * n bf16
    words through its data pointer, so it must be exactly that."""
    torch = _torch()
    if out is None:
        return torch.empty((m, n), dtype=torch.bfloat16, device=device)
    if out.dtype != torch.bfloat16:
        raise TypeError(f"out must be bfloat16, got {out.dtype}")
    if out.device != device:
        raise ValueError(f"out is on {out.device}, the inputs on {device}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if tuple(out.shape) not in ((m, n), tuple(lead) + (n,)):
        raise ValueError(f"out must have shape {(m, n)} or {tuple(lead) + (n,)}, got {tuple(out.shape)}")
    return out


def _workspace(workspace, need: int, device):
    """A caller's workspace, or a new one: contiguous uint8 bytes on the
    inputs' device (its size is checked by the library)."""
    torch = _torch()
    if workspace is None:
        return torch.empty((max(need, 1),), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {workspace.dtype}")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, the inputs on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace


def sparsify_2of4(x, fold_scale: bool = False, with_scale: bool = True):
    """Mask, compensation scale and canonical compression of x [..., K].

    Returns (vals [M, K/2] bf16, idx [M, ceil(K/8)] uint8, scale [M] fp32 or None).
    """
    torch = _torch()
    x2 = _as_2d(x, "x")
    m, k = x2.shape
    vals = torch.empty((m, k // 2), dtype=torch.bfloat16, device=x2.device)
    idx = torch.empty((m, (k // 4 + 1) // 2), dtype=torch.uint8, device=x2.device)
    scale = torch.empty((m,), dtype=torch.float32, device=x2.device) if with_scale else None
    with _on(x2.device):
        st = lib().rtl_sparsify_2of4(x2.data_ptr(), m, k, vals.data_ptr(), idx.data_ptr(),
                                     scale.data_ptr() if scale is not None else None,
                                     FOLD_SCALE if fold_scale else 0, _stream())
    _check(st, "rtl_sparsify_2of4")
    return vals, idx, scale


def sparse_linear(x, w, lora_a=None, lora_b=None, lora_scale: float = 1.0, out=None, workspace=None):
    """Y = S(X) W^T + lora_scale * ((X - S(X)) A^T) B^T for x [..., K], w [N, K],
    lora_a [r, K], lora_b [N, r] (bf16, device).  Returns y [..., N] bf16."""
    x2 = _as_2d(x, "x")
    w2 = _as_2d(w, "w")
    m, k = x2.shape
    n = w2.shape[0]
    if w2.shape[1] != k:
        raise ValueError(f"w has {w2.shape[1]} input channels, x has {k}")
    r = 0
    if lora_a is not None or lora_b is not None:
        if lora_a is None or lora_b is None:
            raise ValueError("lora_a and lora_b go together")
        lora_a = _as_2d(lora_a, "lora_a")
        lora_b = _as_2d(lora_b, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape[1] != k or lora_b.shape != (n, r):
            raise ValueError(f"LoRA shapes {tuple(lora_a.shape)}, {tuple(lora_b.shape)} do not match "
                             f"K={k}, N={n}")
    y = _out(out, m, n, x.shape[:-1], x2.device)
    workspace = _workspace(workspace, sparse_linear_workspace_bytes(m, k, r), x2.device)
    with _on(x2.device, w=w2, lora_a=lora_a, lora_b=lora_b):
        st = lib().rtl_sparse_linear(
            x2.data_ptr(), w2.data_ptr(),
            lora_a.data_ptr() if r else None, lora_b.data_ptr() if r else None,
            m, n, k, r, float(lora_scale), y.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "rtl_sparse_linear")
    return y.reshape(*x.shape[:-1], n)


def sparse_linear_noalloc(x, w, lora_a=None, lora_b=None, lora_scale: float = 1.0, out=None):
    """sparse_linear without a workspace (rtl_sparse_linear_noalloc): the
    library's fixed per-GPU scratch array (NOALLOC_SCRATCH_BYTES) stands in
    for it, so with ``out`` given nothing is allocated.  Calls that can
    overlap on one GPU share that array and must be serialised."""
    x2 = _as_2d(x, "x")
    w2 = _as_2d(w, "w")
    m, k = x2.shape
    n = w2.shape[0]
    if w2.shape[1] != k:
        raise ValueError(f"w has {w2.shape[1]} input channels, x has {k}")
    r = 0
    if lora_a is not None or lora_b is not None:
        if lora_a is None or lora_b is None:
            raise ValueError("lora_a and lora_b go together")
        lora_a = _as_2d(lora_a, "lora_a")
        lora_b = _as_2d(lora_b, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape[1] != k or lora_b.shape != (n, r):
            raise ValueError(f"LoRA shapes {tuple(lora_a.shape)}, {tuple(lora_b.shape)} do not match "
                             f"K={k}, N={n}")
    y = _out(out, m, n, x.shape[:-1], x2.device)
    with _on(x2.device, w=w2, lora_a=lora_a, lora_b=lora_b):
        st = lib().rtl_sparse_linear_noalloc(
            x2.data_ptr(), w2.data_ptr(), lora_a.data_ptr() if r else None, lora_b.data_ptr() if r else None,
            m, n, k, r, float(lora_scale), y.data_ptr(), _stream())
    _check(st, "rtl_sparse_linear_noalloc")
    return y.reshape(*x.shape[:-1], n)


class Prepared:
    """Workspace filled by ``prepare``: the compressed activation, the
    per-token scale and the LoRA-down product of one x, reusable by ``apply``
    against any number of weights with the same K."""

    def __init__(self, workspace, m: int, k: int, r: int, lead_shape):
        self.workspace, self.m, self.k, self.r, self.lead_shape = workspace, m, k, r, lead_shape


def prepare(x, lora_a=None, lora_scale: float = 1.0, workspace=None, variant: int = 0) -> Prepared:
    """First half of sparse_linear: reads x once (rtl_sparse_linear_prepare,
    or rtl_sparse_linear_prepare_variant for a nonzero ``variant``: one of
    COMP_* | one of LORA_*)."""
    x2 = _as_2d(x, "x")
    m, k = x2.shape
    r = 0
    if lora_a is not None:
        lora_a = _as_2d(lora_a, "lora_a")
        r = lora_a.shape[0]
        if lora_a.shape[1] != k:
            raise ValueError(f"lora_a has {lora_a.shape[1]} input channels, x has {k}")
    workspace = _workspace(workspace, sparse_linear_workspace_bytes(m, k, r), x2.device)
    with _on(x2.device, lora_a=lora_a):
        if variant:
            st = lib().rtl_sparse_linear_prepare_variant(x2.data_ptr(), lora_a.data_ptr() if r else None, m, k,
                                                         r, float(lora_scale), int(variant), workspace.data_ptr(),
                                                         workspace.numel(), _stream())
        else:
            st = lib().rtl_sparse_linear_prepare(x2.data_ptr(), lora_a.data_ptr() if r else None, m, k, r,
                                                 float(lora_scale), workspace.data_ptr(), workspace.numel(),
                                                 _stream())
    _check(st, "rtl_sparse_linear_prepare_variant" if variant else "rtl_sparse_linear_prepare")
    return Prepared(workspace, m, k, r, tuple(x.shape[:-1]))


def apply(prep: Prepared, w, lora_b=None, out=None):
    """Second half of sparse_linear: sparse GEMM + scale + LoRA-up (rtl_sparse_linear_apply)."""
    w2 = _as_2d(w, "w")
    n = w2.shape[0]
    if w2.shape[1] != prep.k:
        raise ValueError(f"w has {w2.shape[1]} input channels, the prepared x has {prep.k}")
    if prep.r:
        if lora_b is None:
            raise ValueError("the prepared x carries a LoRA branch: lora_b is required")
        lora_b = _as_2d(lora_b, "lora_b")
        if tuple(lora_b.shape) != (n, prep.r):
            raise ValueError(f"lora_b must be [{n}, {prep.r}], got {tuple(lora_b.shape)}")
    if w2.device != prep.workspace.device:
        raise ValueError(f"w is on {w2.device}, the prepared activation on {prep.workspace.device}")
    y = _out(out, prep.m, n, prep.lead_shape, w2.device)
    with _on(w2.device, lora_b=lora_b if prep.r else None):
        st = lib().rtl_sparse_linear_apply(prep.workspace.data_ptr(), prep.workspace.numel(), w2.data_ptr(),
                                           lora_b.data_ptr() if prep.r else None, prep.m, n, prep.k, prep.r,
                                           y.data_ptr(), _stream())
    _check(st, "rtl_sparse_linear_apply")
    return y.reshape(*prep.lead_shape, n)


def sparse_linear_compressed(vals, idx, scale, w, out=None, workspace=None):
    """Y = scale * (decompress(vals, idx) W^T) for an activation compressed by
    ``sparsify_2of4`` (vals [M, K/2] bf16, idx [M, ceil(K/8)] uint8, scale [M]
    fp32 or None), w [N, K] bf16.  Returns y [M, N] bf16."""
    torch = _torch()
    v2 = _as_2d(vals, "vals")
    w2 = _as_2d(w, "w")
    m = v2.shape[0]
    n, k = w2.shape
    if v2.shape[1] * 2 != k:
        raise ValueError(f"vals has {v2.shape[1]} columns, w has {k} input channels")
    if idx.dtype != torch.uint8 or not idx.is_cuda or not idx.is_contiguous() or \
            tuple(idx.shape) != (m, (k // 4 + 1) // 2):
        raise ValueError("idx must be a contiguous uint8 device tensor [M, ceil(K/8)]")
    if scale is not None and (scale.dtype != torch.float32 or not scale.is_cuda or scale.numel() != m):
        raise ValueError("scale must be a float32 device tensor [M] or None")
    y = _out(out, m, n, (m,), w2.device)
    workspace = _workspace(workspace, sparse_linear_workspace_bytes(m, k, 0), w2.device)
    with _on(w2.device, vals=v2, idx=idx, scale=scale):
        st = lib().rtl_sparse_linear_compressed(v2.data_ptr(), idx.data_ptr(),
                                                scale.data_ptr() if scale is not None else None,
                                                w2.data_ptr(), m, n, k, y.data_ptr(), workspace.data_ptr(),
                                                workspace.numel(), _stream())
    _check(st, "rtl_sparse_linear_compressed")
    return y


def dense_linear(x, w, out=None):
    """Y = X W^T on the dense matrix cores (the baseline)."""
    x2 = _as_2d(x, "x")
    w2 = _as_2d(w, "w")
    m, k = x2.shape
    n = w2.shape[0]
    if w2.shape[1] != k:
        raise ValueError(f"w has {w2.shape[1]} input channels, x has {k}")
    y = _out(out, m, n, x.shape[:-1], x2.device)
    with _on(x2.device, w=w2):
        st = lib().rtl_dense_linear(x2.data_ptr(), w2.data_ptr(), m, n, k, y.data_ptr(), _stream())
    _check(st, "rtl_dense_linear")
    return y.reshape(*x.shape[:-1], n)
