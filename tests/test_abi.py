"""The C-ABI library on the host, without a GPU: it loads, exports every
symbol include/*.h declares, and rejects every invalid argument with its
documented status before any HIP call.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import activation_sparse_gemm_token_amd as rtl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtlynx.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, NULLP, SHAPE, MISAL, WS, NODEV, ARCH, HIP, FLAGS = range(9)
P = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
P2 = 0x20000
P3 = 0x30000
P4 = 0x40000
P5 = 0x50000
WSP = 0x60000
BIG = 1 << 40


def _declared_symbols():
    """Every rtl_ function named in include/*.h (declarations and the
    comments that name them)."""
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"\b(rtl_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = rtl.lib()
    syms = _declared_symbols()
    assert set(syms) >= {"rtl_sparsify_2of4", "rtl_sparse_linear", "rtl_dense_linear",
                         "rtl_sparse_linear_workspace_bytes", "rtl_status_string", "rtl_version"}
    for s in syms:
        assert hasattr(lib, s), s


def test_only_declared_symbols_are_exported():
    """-fvisibility=hidden: the C ABI is the whole dynamic interface."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", rtl.library_path], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    rtl_syms = {s for s in exported if s.startswith("rtl_")}
    assert rtl_syms == set(_declared_symbols())


def test_version_and_status_strings():
    assert rtl.version() == 10000
    for code in range(10):
        s = rtl.status_string(code)
        assert isinstance(s, str) and s
    assert rtl.status_string(OK) == "ok"
    assert rtl.status_string(99) == "unknown status"


def test_workspace_bytes():
    # rows padded to 256, K to 128, r to 32; regions 256-byte aligned
    def expect(m, k, r):
        mp, kp, rp = -(-m // 256) * 256, -(-k // 128) * 128, -(-r // 32) * 32
        up = lambda v: -(-v // 256) * 256
        o = up(mp * kp)
        o = up(o + mp * kp // 8)
        o = up(o + mp * 4)
        return up(o + mp * rp * 4)
    for m, k, r in [(1, 4, 0), (64, 256, 8), (4096, 3072, 64), (9216, 3072, 64), (300, 516, 24), (257, 1000, 5)]:
        assert rtl.sparse_linear_workspace_bytes(m, k, r) == expect(m, k, r)
    assert rtl.sparse_linear_workspace_bytes(0, 256, 8) == 0
    for bad in [(-1, 256, 8), (64, 6, 8), (64, 0, 8), (64, 256, -1), (64, 256, 129), (64, 2, 0),
                (1, 1 << 29, 0), (1 << 22, 256, 0)]:
        assert rtl.sparse_linear_workspace_bytes(*bad) == 0


def _sl(x=P, w=P2, a=P3, b=P4, m=64, n=128, k=256, r=8, alpha=1.0, y=P5, ws=WSP, wsb=BIG, stream=None):
    return rtl.lib().rtl_sparse_linear(x, w, a, b, m, n, k, r, alpha, y, ws, wsb, stream)


def _sp(x=P, m=64, k=256, vals=P2, idx=P3, scale=P4, flags=0, stream=None):
    return rtl.lib().rtl_sparsify_2of4(x, m, k, vals, idx, scale, flags, stream)


def _dl(x=P, w=P2, m=64, n=128, k=256, y=P3, stream=None):
    return rtl.lib().rtl_dense_linear(x, w, m, n, k, y, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(k=0), SHAPE), (dict(k=2), SHAPE), (dict(m=-1), SHAPE),
    (dict(n=-5), SHAPE), (dict(r=-1), SHAPE), (dict(r=129), SHAPE), (dict(k=1 << 31), SHAPE),
    (dict(x=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP),
    (dict(a=None), NULLP), (dict(b=None), NULLP),
    (dict(x=P + 8), MISAL), (dict(w=P2 + 2), MISAL), (dict(y=P5 + 4), MISAL),
    (dict(a=P3 + 8), MISAL), (dict(b=P4 + 8), MISAL),
    (dict(ws=None), WS), (dict(wsb=1024), WS), (dict(ws=WSP + 8), MISAL),
    (dict(m=0), OK), (dict(n=0), OK), (dict(m=0, x=None, y=None), OK),
    # 32-bit buffer offsets: every tensor below 2 GiB
    (dict(m=1 << 22, k=256), SHAPE), (dict(n=1 << 22, k=256), SHAPE), (dict(m=1 << 15, n=1 << 15), SHAPE),
    (dict(m=1, n=1, k=1 << 30, r=0), SHAPE), (dict(n=1 << 24, r=64), SHAPE),
])
def test_sparse_linear_rejects_invalid_arguments(kw, status):
    assert _sl(**kw) == status


def test_sparse_linear_workspace_exact_size_passes_validation():
    need = rtl.sparse_linear_workspace_bytes(64, 256, 8)
    st = _sl(wsb=need - 1)
    assert st == WS
    if _no_gpu():
        assert _sl(wsb=need) == NODEV


def test_sparse_linear_r0_ignores_lora_pointers():
    if _no_gpu():
        assert _sl(r=0, a=None, b=None) == NODEV
        assert _sl(r=0, a=P3 + 8, b=None) == NODEV     # ignored, so not MISALIGNED


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(m=-1), SHAPE), (dict(k=0), SHAPE),
    (dict(x=None), NULLP), (dict(vals=None), NULLP), (dict(idx=None), NULLP),
    (dict(x=P + 8), MISAL), (dict(vals=P2 + 4), MISAL), (dict(idx=P3 + 1), MISAL), (dict(scale=P4 + 4), MISAL),
    (dict(flags=2), FLAGS), (dict(flags=0xFFFF), FLAGS),
    (dict(m=0), OK), (dict(m=0, x=None), OK),
])
def test_sparsify_rejects_invalid_arguments(kw, status):
    assert _sp(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(m=-1), SHAPE), (dict(n=-1), SHAPE),
    (dict(x=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP),
    (dict(x=P + 8), MISAL), (dict(w=P2 + 8), MISAL), (dict(y=P3 + 2), MISAL),
    (dict(m=0), OK), (dict(n=0), OK),
])
def test_dense_linear_rejects_invalid_arguments(kw, status):
    assert _dl(**kw) == status


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def test_valid_calls_without_a_device_report_no_device():
    """With valid arguments the only thing missing here is the GPU."""
    if not _no_gpu():
        pytest.skip("a GPU is present: valid calls would launch on fake pointers")
    assert _sp() == NODEV
    assert _sp(scale=None, flags=1) == NODEV
    assert _sl() == NODEV
    assert _dl() == NODEV
    # just below the 2 GiB limit: Y and its last tile's padding rows = 2^31 - 2^18 bytes
    assert _dl(m=(1 << 14) - 256, n=(1 << 16) - 8) == NODEV
    assert _dl(m=1 << 14, n=1 << 16) == SHAPE
    # the library stays usable after errors
    assert _sl(k=6) == SHAPE
    assert _sl() == NODEV


def test_python_wrappers_reject_bad_tensors():
    import torch
    x = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        rtl.sparse_linear(x, x)
    xb = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rtl.dense_linear(xb, xb)          # host tensors


def _na(x=P, w=P2, a=P3, b=P4, m=64, n=128, k=256, r=8, alpha=1.0, y=P5, stream=None):
    return rtl.lib().rtl_sparse_linear_noalloc(x, w, a, b, m, n, k, r, alpha, y, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(m=-1), SHAPE), (dict(r=129), SHAPE),
    (dict(x=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP), (dict(a=None), NULLP),
    (dict(x=P + 8), MISAL), (dict(b=P4 + 8), MISAL), (dict(m=0), OK), (dict(n=0), OK),
    # the layer's workspace must fit the fixed scratch array (64 MiB)
    (dict(m=8192, k=8192, r=64), WS), (dict(m=1 << 14, k=4096, r=0), WS),
])
def test_noalloc_rejects_invalid_arguments(kw, status):
    assert _na(**kw) == status


def test_noalloc_limit_is_the_workspace_size():
    """Largest accepted layers: workspace just within RTL_NOALLOC_SCRATCH_BYTES."""
    lim = rtl.NOALLOC_SCRATCH_BYTES
    assert rtl.sparse_linear_workspace_bytes(9216, 3072, 64) <= lim
    assert rtl.sparse_linear_workspace_bytes(4096, 12288, 64) <= lim
    assert rtl.sparse_linear_workspace_bytes(8192, 8192, 64) > lim
    if _no_gpu():
        assert _na(m=9216, k=3072, r=64) == NODEV
        assert _na(m=4096, k=12288, r=64) == NODEV
        assert _na(r=0, a=None, b=None) == NODEV


def test_output_and_workspace_checks():
    """A caller's out= must be exactly the bf16 [M, N] (or [..., N]) block the
    kernels write, on the inputs' device; a caller's workspace contiguous
    uint8 bytes on that device."""
    import torch
    cpu = torch.device("cpu")
    good = torch.zeros(6, 8, dtype=torch.bfloat16)
    assert rtl._out(good, 6, 8, (6,), cpu) is good
    assert rtl._out(torch.zeros(2, 3, 8, dtype=torch.bfloat16), 6, 8, (2, 3), cpu).shape == (2, 3, 8)
    assert rtl._out(None, 6, 8, (6,), cpu).shape == (6, 8)
    for bad, exc in [(torch.zeros(6, 8, dtype=torch.float32), TypeError),
                     (torch.zeros(5, 8, dtype=torch.bfloat16), ValueError),
                     (torch.zeros(6, 9, dtype=torch.bfloat16), ValueError),
                     (torch.zeros(48, dtype=torch.bfloat16), ValueError),
                     (torch.zeros(8, 6, dtype=torch.bfloat16).t(), ValueError),
                     (torch.zeros(6, 8, dtype=torch.bfloat16, device="meta"), ValueError)]:
        with pytest.raises(exc):
            rtl._out(bad, 6, 8, (6,), cpu)
    ws = torch.zeros(1024, dtype=torch.uint8)
    assert rtl._workspace(ws, 512, cpu) is ws
    assert rtl._workspace(None, 512, cpu).numel() == 512
    for bad, exc in [(torch.zeros(256, dtype=torch.float32), TypeError),
                     (torch.zeros(1024, dtype=torch.uint8, device="meta"), ValueError),
                     (torch.zeros(2048, dtype=torch.uint8)[::2], ValueError)]:
        with pytest.raises(exc):
            rtl._workspace(bad, 512, cpu)


def _pr(x=P, a=P2, m=64, k=256, r=8, alpha=1.0, ws=WSP, wsb=BIG, stream=None):
    return rtl.lib().rtl_sparse_linear_prepare(x, a, m, k, r, alpha, ws, wsb, stream)


def _ap(ws=WSP, wsb=BIG, w=P, b=P2, m=64, n=128, k=256, r=8, y=P3, stream=None):
    return rtl.lib().rtl_sparse_linear_apply(ws, wsb, w, b, m, n, k, r, y, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(r=129), SHAPE), (dict(m=-2), SHAPE),
    (dict(x=None), NULLP), (dict(a=None), NULLP), (dict(x=P + 8), MISAL), (dict(a=P2 + 8), MISAL),
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(ws=WSP + 4), MISAL), (dict(m=0), OK),
    (dict(m=1, k=1 << 29, r=0), SHAPE),        # X is 1 GiB, but the padded workspace is 128 GiB
])
def test_prepare_rejects_invalid_arguments(kw, status):
    assert _pr(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(n=-1), SHAPE), (dict(r=200), SHAPE),
    (dict(w=None), NULLP), (dict(b=None), NULLP), (dict(y=None), NULLP),
    (dict(w=P + 8), MISAL), (dict(b=P2 + 8), MISAL), (dict(y=P3 + 2), MISAL),
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(m=0), OK), (dict(n=0), OK),
    (dict(m=1 << 15, n=1 << 15), SHAPE), (dict(n=1 << 23), SHAPE),
])
def test_apply_rejects_invalid_arguments(kw, status):
    assert _ap(**kw) == status


def test_prepare_apply_without_device():
    if not _no_gpu():
        pytest.skip("a GPU is present")
    assert _pr() == NODEV
    assert _ap() == NODEV
    assert _pr(r=0, a=None) == NODEV


def _cl(v=P, i=P2, s=P3, w=P4, m=64, n=128, k=256, y=P5, ws=WSP, wsb=BIG, stream=None):
    return rtl.lib().rtl_sparse_linear_compressed(v, i, s, w, m, n, k, y, ws, wsb, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(k=6), SHAPE), (dict(k=0), SHAPE), (dict(m=-1), SHAPE), (dict(n=-1), SHAPE),
    (dict(v=None), NULLP), (dict(i=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP),
    (dict(v=P + 8), MISAL), (dict(i=P2 + 1), MISAL), (dict(s=P3 + 4), MISAL), (dict(w=P4 + 8), MISAL),
    (dict(y=P5 + 2), MISAL), (dict(ws=None), WS), (dict(wsb=16), WS), (dict(ws=WSP + 4), MISAL),
    (dict(m=0), OK), (dict(n=0), OK), (dict(m=1 << 15, n=1 << 15), SHAPE),
])
def test_compressed_rejects_invalid_arguments(kw, status):
    assert _cl(**kw) == status


def test_compressed_without_device():
    if not _no_gpu():
        pytest.skip("a GPU is present")
    assert _cl() == NODEV
    assert _cl(s=None) == NODEV           # no scale: s = 1
    need = rtl.lib().rtl_sparse_linear_workspace_bytes(64, 256, 0)
    assert _cl(wsb=need) == NODEV
    assert _cl(wsb=need - 1) == WS


def _pv(x=P, a=P2, m=64, k=256, r=8, alpha=1.0, variant=0x6, ws=WSP, wsb=BIG, stream=None):
    return rtl.lib().rtl_sparse_linear_prepare_variant(x, a, m, k, r, alpha, variant, ws, wsb, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(variant=0x10), FLAGS), (dict(variant=0xC), FLAGS), (dict(variant=0x80000000), FLAGS),
    (dict(k=6), SHAPE), (dict(r=129), SHAPE), (dict(x=None), NULLP), (dict(a=None), NULLP),
    (dict(x=P + 8), MISAL), (dict(ws=None), WS), (dict(wsb=16), WS), (dict(m=0), OK),
])
def test_prepare_variant_rejects_invalid_arguments(kw, status):
    assert _pv(**kw) == status


def test_prepare_variant_without_device():
    if not _no_gpu():
        pytest.skip("a GPU is present")
    for comp in (rtl.COMP_TOKEN, rtl.COMP_NONE, rtl.COMP_TENSOR, rtl.COMP_GROUP):
        for lora in (rtl.LORA_RESIDUAL, rtl.LORA_PRUNED, rtl.LORA_INPUT):
            assert _pv(variant=comp | lora) == NODEV
