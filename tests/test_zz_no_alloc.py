"""rtl_sparse_linear_noalloc, the entry point for callers that cannot
allocate (HIP graph capture, tight serving loops, harnesses that forbid
hipMalloc), against rtl_sparse_linear with a caller workspace: bit for bit,
on two calls in a row, the second on a smaller layer (the fixed scratch array
keeps the first call's contents), and through the C ABI."""
import ctypes
import sys

import numpy as np
import pytest

from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import activation_sparse_gemm_token_amd as rtl  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _layer(m, k, n, r, seed):
    rng = np.random.default_rng(seed)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01) if r else None
    b = gen.gaussian_bits(rng, (n, r), 0.01) if r else None
    return [None if t is None else to_dev(t) for t in (x, w, a, b)]


def _noalloc_abi(x, w, a, b, alpha, y):
    """The C entry point itself, arguments marshalled by hand."""
    m, k = x.shape
    n = w.shape[0]
    r = 0 if a is None else a.shape[0]
    fn = rtl.lib().rtl_sparse_linear_noalloc
    st = fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
            ctypes.c_void_p(a.data_ptr() if r else None), ctypes.c_void_p(b.data_ptr() if r else None),
            ctypes.c_int64(m), ctypes.c_int64(n), ctypes.c_int64(k), ctypes.c_int64(r), ctypes.c_float(alpha),
            ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, rtl.status_string(st)


CASES = [
    # (first layer, second smaller layer): headline, then a ragged one with a
    # channel tail; the largest DMA pre-pass layer, then a generic pre-pass one
    ((4096, 3072, 12288, 64), (300, 520, 200, 24)),
    ((4096, 12288, 3072, 64), (257, 1028, 333, 96)),
    ((9216, 3072, 3072, 64), (64, 256, 128, 0)),
]


@pytest.mark.parametrize("pair", CASES, ids=lambda p: "_".join("x".join(map(str, s)) for s in p))
def test_noalloc_matches_workspace_entry_point(pair):
    for i, (m, k, n, r) in enumerate(pair):
        say(f"[no-alloc] call {i}: M={m} K={k} N={n} r={r}")
        x, w, a, b = _layer(m, k, n, r, seed=m + k + n + r)
        want = rtl.sparse_linear(x, w, a, b, 0.5)
        y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        _noalloc_abi(x, w, a, b, 0.5, y)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), to_host(want)), f"call {i} {(m, k, n, r)} differs"
        y2 = rtl.sparse_linear_noalloc(x, w, a, b, 0.5)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y2), to_host(want)), f"binding, call {i} {(m, k, n, r)} differs"


def test_noalloc_rejects_a_layer_beyond_the_scratch():
    x = torch.zeros((8192, 8192), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((64, 8192), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rtl.RtlError) as e:
        rtl.sparse_linear_noalloc(x, w)
    assert e.value.status == 4
