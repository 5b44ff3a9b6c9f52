"""GPU parity at the largest tensors the C ABI admits.

Every byte offset the kernels form is a 32-bit buffer offset, and the host
admits a call only while each tensor, with the 256 rows past its end that
the last tile addresses, and each workspace region stay below 2 GiB.  One
case puts each of Y, X (and with it the workspace's operand region) and W
within a few MiB of that bound, with ragged M, N and K, and compares Y on
sampled rows and columns with the oracle (an output element depends only on
its row of X and its column of W, so the oracle runs on those alone).  The
sampled rows include the last ones, whose offsets are the largest.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import activation_sparse_gemm_token_amd as rtl  # noqa: E402

DEV = "cuda:0"
LIMIT = 1 << 31

# (M, K, N, r, what): (M + 256) N 2, (M + 256) K 2 and (N + 256) K 2 bytes
# each below 2^31; the named tensor within 3 MiB of it.
CASES = [
    (32504, 520, 32768, 64, "Y"),
    (65240, 16384, 264, 64, "X"),
    (300, 16384, 65256, 32, "W"),
]


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-{c[0]}x{c[1]}x{c[2]}")
def test_largest_admitted_tensors(case):
    m, k, n, r, what = case
    big = {"Y": (m + 256) * n * 2, "X": (m + 256) * k * 2, "W": (n + 256) * k * 2}[what]
    assert LIMIT - (3 << 20) < big < LIMIT, "the case must sit just below the 2 GiB bound"
    print(f"[max-size] {what} near 2 GiB: M={m} K={k} N={n} r={r}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(m + k + n)
    x = gen.uniform_bits(rng, (m, k), emax=1)
    w = gen.uniform_bits(rng, (n, k), emax=-5)
    a = gen.uniform_bits(rng, (r, k), emax=-6)
    b = gen.uniform_bits(rng, (n, r), emax=-6)
    xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
    y = rtl.sparse_linear(xd, wd, ad, bd, 0.5)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(16), np.arange(m - 40, m), rng.integers(0, m, 24),
                                     255 + 256 * np.arange(0, m // 256, max(1, m // 256 // 8))]))
    rows = rows[rows < m]
    cols = np.unique(np.concatenate([np.arange(8), np.arange(n - 24, n), rng.integers(0, n, 96)]))
    got = oracle.bf16_bits_to_f64(
        y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]
        .contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    ref = oracle.sparse_linear_ref(x[rows], w[cols], a, b[cols], 0.5)
    tol = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    if (err > tol).any():
        i, j = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {int((err > tol).sum())} elements out of tolerance; worst at row "
                             f"{rows[i]} column {cols[j]}: got {got[i, j]!r} want {ref[i, j]!r}")
    del xd, wd, ad, bd, y
    torch.cuda.empty_cache()
