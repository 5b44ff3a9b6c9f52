"""Selective layer skipping (rtl_layer_linear, include/rtlynx_layers.h).

The RT-Lynx pages skip the online sparsification on some sensitive layers of
single-stream diffusion transformers, or give different layers different
sparsification strategies (ai-feeds summary, 方法 / 核心模块 3; qingkeai
article, section 03, item 3).  A ``LayerPolicy`` holds one mode per layer --
``DENSE`` (skipped: the dense product, which is what the layer computes
without sparsification, the LoRA branch then having no residual to act on) or
a sparsification variant (``COMP_* | LORA_*``; 0 is the default layer) -- and
``policy.linear(layer, ...)`` runs one layer through the C dispatch.
``STREAM_W`` OR-ed into a sparse layer's mode marks its weights as not
expected in the caches (each layer of a model running once per forward
pass): its GEMM then probes the weight lines into L2 ahead of their copies,
with the same output bits.  Argument marshalling only, as in the package's
other bindings.
"""
from __future__ import annotations

import ctypes

from . import _as_2d, _check, _on, _out, _stream, _workspace, lib, sparse_linear_workspace_bytes

DENSE = 0x100
STREAM_W = 0x200

_c_i64, _c_vp = ctypes.c_int64, ctypes.c_void_p
_SIG = (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp,
                       _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_vp, _c_vp, ctypes.c_size_t, _c_vp])


def _fn():
    fn = lib().rtl_layer_linear
    fn.restype, fn.argtypes = _SIG
    return fn


class LayerPolicy:
    """Per-layer modes of a model with ``num_layers`` sparsifiable linear
    layers: every layer sparse (variant 0) unless listed in ``dense`` or
    given a variant in ``variants``; ``stream_weights`` (True for every
    layer, or an iterable of layers) adds the ``STREAM_W`` hint."""

    def __init__(self, num_layers: int, dense=(), variants=None, stream_weights=()):
        if num_layers < 0:
            raise ValueError("num_layers must be >= 0")
        self.modes = (ctypes.c_uint32 * max(num_layers, 1))()
        self.num_layers = num_layers
        for layer, v in (variants or {}).items():
            self.modes[self._index(layer)] = int(v)
        for layer in dense:
            self.modes[self._index(layer)] = DENSE
        if stream_weights is True:
            stream_weights = range(num_layers)
        for layer in stream_weights or ():
            self.modes[self._index(layer)] |= STREAM_W

    def _index(self, layer: int) -> int:
        if not 0 <= layer < self.num_layers:
            raise IndexError(f"layer {layer} outside [0, {self.num_layers})")
        return layer

    def mode(self, layer: int) -> int:
        return int(self.modes[self._index(layer)])

    def linear(self, layer: int, x, w, lora_a=None, lora_b=None, lora_scale: float = 1.0, out=None,
               workspace=None):
        """Layer ``layer`` on x [..., K] with weight w [N, K] and LoRA factors
        (used by sparse layers only).  Returns y [..., N] bf16."""
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
            if lora_a.shape[1] != k or tuple(lora_b.shape) != (n, r):
                raise ValueError(f"LoRA shapes {tuple(lora_a.shape)}, {tuple(lora_b.shape)} do not match "
                                 f"K={k}, N={n}")
        y = _out(out, m, n, x.shape[:-1], x2.device)
        if self.mode(layer) & ~STREAM_W != DENSE:
            workspace = _workspace(workspace, sparse_linear_workspace_bytes(m, k, r), x2.device)
        with _on(x2.device, w=w2, lora_a=lora_a, lora_b=lora_b):
            st = _fn()(self.modes, self.num_layers, layer, x2.data_ptr(), w2.data_ptr(),
                       lora_a.data_ptr() if r else None, lora_b.data_ptr() if r else None, m, n, k, r,
                       float(lora_scale), y.data_ptr(), workspace.data_ptr() if workspace is not None else None,
                       workspace.numel() if workspace is not None else 0, _stream())
        _check(st, "rtl_layer_linear")
        return y.reshape(*x.shape[:-1], n)
