"""rtl_layer_linear on the host, without a GPU: the per-layer dispatch of
selective layer skipping validates the layer table and the mode before any
HIP call, and hands valid calls to the dense or the sparse entry point (which
then report that no device is present)."""
import ctypes
import os
import re

import pytest

import activation_sparse_gemm_token_amd as rtl
from activation_sparse_gemm_token_amd import layers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtlynx_layers.h")
OK, NULLP, SHAPE, MISAL, WS, NODEV, ARCH, HIP, FLAGS = range(9)
P, P2, P3, P4, P5, WSP = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000
BIG = 1 << 40


def _modes(*vals):
    return (ctypes.c_uint32 * len(vals))(*vals)


def _ll(modes, n, layer, x=P, w=P2, a=P3, b=P4, m=64, nn=128, k=256, r=8, y=P5, ws=WSP, wsb=BIG):
    return layers._fn()(modes, n, layer, x, w, a, b, m, nn, k, r, 1.0, y, ws, wsb, None)


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def test_header_symbol_is_exported():
    syms = set(re.findall(r"\b(rtl_[a-z0-9_]+)\s*\(", open(HEADER).read()))
    assert "rtl_layer_linear" in syms
    for s in syms:
        assert hasattr(rtl.lib(), s), s


def test_rejects_bad_tables_and_modes():
    m = _modes(0, layers.DENSE, rtl.COMP_NONE | rtl.LORA_PRUNED)
    assert _ll(m, 3, 3) == SHAPE
    assert _ll(m, 3, -1) == SHAPE
    assert _ll(m, -1, 0) == SHAPE
    assert _ll(None, 3, 0) == NULLP
    assert _ll(_modes(0x10), 1, 0) == FLAGS
    assert _ll(_modes(0xC), 1, 0) == FLAGS          # LoRA-input field 3 is no variant
    assert _ll(_modes(0x101), 1, 0) == FLAGS        # dense is not combined with a variant
    assert _ll(_modes(0x400), 1, 0) == FLAGS        # no such hint
    assert _ll(_modes(layers.STREAM_W | 0xC), 1, 0) == FLAGS
    assert _ll(_modes(layers.STREAM_W | 0x101), 1, 0) == FLAGS


def test_stream_hint_is_accepted_on_every_mode():
    for mode in (0, rtl.COMP_GROUP | rtl.LORA_INPUT, layers.DENSE):
        ms = _modes(mode | layers.STREAM_W)
        assert _ll(ms, 1, 0, k=6) == SHAPE
        assert _ll(ms, 1, 0, y=P5 + 2) == MISAL
        if mode != layers.DENSE:
            assert _ll(ms, 1, 0, wsb=16) == WS
        if _no_gpu():
            assert _ll(ms, 1, 0) == NODEV


def test_sparse_modes_validate_like_the_sparse_path():
    for mode in (0, rtl.COMP_GROUP | rtl.LORA_INPUT):
        ms = _modes(mode)
        assert _ll(ms, 1, 0, k=6) == SHAPE
        assert _ll(ms, 1, 0, w=None) == NULLP
        assert _ll(ms, 1, 0, y=P5 + 2) == MISAL
        assert _ll(ms, 1, 0, b=P4 + 8) == MISAL
        assert _ll(ms, 1, 0, wsb=16) == WS
        assert _ll(ms, 1, 0, nn=1 << 23) == SHAPE
        assert _ll(ms, 1, 0, m=0) == OK


def test_dense_mode_ignores_lora_and_workspace():
    md = _modes(layers.DENSE)
    assert _ll(md, 1, 0, k=6) == SHAPE
    assert _ll(md, 1, 0, x=None) == NULLP
    if _no_gpu():
        assert _ll(md, 1, 0, a=None, b=None, ws=None, wsb=0) == NODEV
        assert _ll(_modes(0), 1, 0) == NODEV
        assert _ll(_modes(rtl.COMP_TENSOR), 1, 0) == NODEV


def test_policy_object():
    p = layers.LayerPolicy(5, dense=(1, 3), variants={2: rtl.COMP_NONE | rtl.LORA_PRUNED})
    assert [p.mode(i) for i in range(5)] == [0, layers.DENSE, rtl.COMP_NONE | rtl.LORA_PRUNED, layers.DENSE, 0]
    with pytest.raises(IndexError):
        p.mode(5)
    with pytest.raises(IndexError):
        layers.LayerPolicy(2, dense=(2,))
    s = layers.LayerPolicy(3, dense=(1,), stream_weights=True)
    assert [s.mode(i) for i in range(3)] == [layers.STREAM_W, layers.DENSE | layers.STREAM_W, layers.STREAM_W]
    s = layers.LayerPolicy(3, variants={0: rtl.COMP_NONE}, stream_weights=(0, 2))
    assert [s.mode(i) for i in range(3)] == [rtl.COMP_NONE | layers.STREAM_W, 0, layers.STREAM_W]
