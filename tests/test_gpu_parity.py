"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars (from the bf16 rounding of the output and the fp32 reductions):
* masks / positions (idx) and unscaled compressed values: bit-exact;
* per-token scale: |s - s_ref| <= 1e-5 s_ref;
* layer output: |Y - Y_ref| <= 1e-2 |Y_ref| + 1e-3 rms(Y_ref), elementwise;
* folded values (RTL_FOLD_SCALE): within one bf16 ulp of s * x.

Every shape, the six full workload sizes included, is compared element by
element in full: every mask, value and scale, every element of Y.
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def y_to_f64(t):
    return oracle.bf16_bits_to_f64(to_host(t))


def assert_y_close(y, ref, what="", rms=None):
    ref = np.asarray(ref, dtype=np.float64)
    if rms is None:
        rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(y - ref)
    tol = 1e-2 * np.abs(ref) + 1e-3 * rms
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst at {i}: "
                             f"y={y[i]!r} ref={ref[i]!r} tol={tol[i]!r} rms={rms!r}")


def check_sparsify(x_bits, fold=False):
    m, k = x_bits.shape
    vals, idx, scale = rtl.sparsify_2of4(to_dev(x_bits), fold_scale=fold)
    torch.cuda.synchronize()
    sx, mask, s_ref, i0, i1 = oracle.sparsify(x_bits)
    v_ref, idx_ref = oracle.compress(x_bits, i0, i1)
    idx_h = idx.cpu().numpy()
    assert np.array_equal(idx_h, idx_ref), "idx (mask) differs"
    s = scale.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(s, s_ref, rtol=1e-5, atol=0)
    vals_h = to_host(vals)
    if not fold:
        assert np.array_equal(vals_h, v_ref), "vals differ"
    else:
        exact = oracle.bf16_bits_to_f64(v_ref) * np.repeat(s_ref, k // 2).reshape(m, k // 2)
        got = oracle.bf16_bits_to_f64(vals_h)
        ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
        assert (np.abs(got - exact) <= ulp).all(), "folded vals beyond one ulp"


def run_sparse_linear(x, w, a, b, alpha=1.0):
    args = [to_dev(x), to_dev(w)]
    if a is not None:
        args += [to_dev(a), to_dev(b)]
    else:
        args += [None, None]
    y = rtl.sparse_linear(*args, lora_scale=alpha)
    torch.cuda.synchronize()
    return y


SMALL_SHAPES = [
    # (M, K, N, r): tiny config, ragged in every dimension, K % 8 == 4, r not a multiple of 8 or 32
    (64, 256, 128, 8),
    (300, 516, 200, 24),
    (257, 1000, 333, 5),
    (1, 4, 1, 1),
    (5, 12, 7, 0),
    (16, 64, 16, 32),
    (512, 3072, 520, 64),
    (33, 260, 300, 128),
    # DMA pre-pass with fewer k-steps than wavefronts (most of them idle):
    # whole k-steps (K = 128) and a channel tail (K = 192 in 4 steps of 64)
    (48, 128, 72, 64),
    (20, 192, 40, 64),
    # rank 128 with K % 8 == 4 over several k-pairs per pre-pass wavefront
    (300, 2052, 200, 128),
    # one and seven tokens against the full headline weight (one row tile,
    # 48 column tiles)
    (1, 3072, 12288, 64),
    (7, 3072, 12288, 64),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_and_ragged_shapes(shape):
    m, k, n, r = shape
    say(f"[parity] shape M={m} K={k} N={n} r={r}")
    rng = np.random.default_rng(m * 7 + k * 3 + n + r)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01) if r else None
    b = gen.gaussian_bits(rng, (n, r), 0.01) if r else None
    check_sparsify(x)
    y = y_to_f64(run_sparse_linear(x, w, a, b, 0.75))
    assert_y_close(y, oracle.sparse_linear_ref(x, w, a, b, 0.75), f"sparse_linear {shape}")
    yd = rtl.dense_linear(to_dev(x), to_dev(w))
    assert_y_close(y_to_f64(yd), oracle.dense_linear_ref(x, w), f"dense_linear {shape}")


def _sweep_shapes(count=24, seed=20261203):
    """Seeded random shapes: K a multiple of 4 (both copy modes, K % 64 of
    every kind), ranks up to the maximum (ranks above 64 take the generic
    pre-pass), N odd or even (unstaged and staged stores), M, N ragged."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(count):
        m = int(rng.integers(1, 600))
        k = 4 * int(rng.integers(1, 320))
        n = int(rng.integers(1, 700))
        r = int(rng.choice([0, 1, 7, 16, 32, 40, 64, 96, 128]))
        shapes.append((m, k, n, r))
    return shapes


@pytest.mark.parametrize("shape", _sweep_shapes(), ids=lambda s: "x".join(map(str, s)))
def test_random_shape_sweep(shape):
    m, k, n, r = shape
    say(f"[parity] sweep M={m} K={k} N={n} r={r}")
    rng = np.random.default_rng(m * 131 + k * 17 + n * 3 + r)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01) if r else None
    b = gen.gaussian_bits(rng, (n, r), 0.01) if r else None
    check_sparsify(x)
    y = y_to_f64(run_sparse_linear(x, w, a, b, 1.25))
    assert_y_close(y, oracle.sparse_linear_ref(x, w, a, b, 1.25), f"sparse_linear {shape}")
    yd = rtl.dense_linear(to_dev(x), to_dev(w))
    assert_y_close(y_to_f64(yd), oracle.dense_linear_ref(x, w), f"dense_linear {shape}")


def test_tiny_config_gather_form():
    x, w, a, b = gen.make_config("tiny")
    y = y_to_f64(run_sparse_linear(x, w, a, b))
    assert_y_close(y, oracle.sparse_linear_gather_ref(x, w, a, b), "tiny vs gather form")


def test_fold_scale_flag():
    rng = np.random.default_rng(4)
    for k in (256, 260):
        check_sparsify(gen.mixture_bernoulli(rng, 40, k), fold=True)


def test_tie_heavy_masks_bit_exact():
    """Values from {0, +-1, +-2, +-4}: most groups hold ties at the keep/prune
    boundary, resolved toward the lower index on both sides."""
    rng = np.random.default_rng(8)
    for k in (256, 1028):
        check_sparsify(gen.tie_heavy(rng, 129, k))


def test_identity_weight_exposes_fused_mask():
    """W = I, r = 0: Y = bf16(s * (M*X)), so the fused kernel's own mask is
    visible as Y != 0 and must equal the oracle's wherever x != 0."""
    rng = np.random.default_rng(12)
    for k in (256, 768):
        x = gen.tie_heavy(rng, 96, k)
        w = gen.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
        y = y_to_f64(run_sparse_linear(x, w, None, None))
        sx, mask, s, _, _ = oracle.sparsify(x)
        nz = oracle.bf16_bits_to_f64(x) != 0
        assert np.array_equal((y != 0)[nz], mask[nz])
        assert_y_close(y, sx, "W = I")


def test_zero_weight_leaves_lora_branch():
    x, w, a, b = gen.make_config("attn_proj", m=256)
    wz = np.zeros((512, x.shape[1]), dtype=np.uint16)
    b = b[:512]
    y = y_to_f64(run_sparse_linear(x, wz, a, b, 1.5))
    assert_y_close(y, oracle.sparse_linear_ref(x, wz, a, b, 1.5), "W = 0")


def test_weight_equal_to_lora_product_gives_dense():
    """W = B A exactly (entries multiples of 2^-6): the sparse layer equals
    the dense product whatever the mask and the scale."""
    rng = np.random.default_rng(21)
    k, n, r = 512, 384, 16
    a = gen.f32_to_bf16_bits(rng.integers(-1, 2, size=(r, k)).astype(np.float32) * 0.125)
    b = gen.f32_to_bf16_bits(rng.integers(-1, 2, size=(n, r)).astype(np.float32) * 0.125)
    wv = oracle.bf16_bits_to_f64(b) @ oracle.bf16_bits_to_f64(a)
    w = gen.f32_to_bf16_bits(wv.astype(np.float32))
    x = gen.mixture_bernoulli(rng, 200, k)
    y = y_to_f64(run_sparse_linear(x, w, a, b, 1.0))
    assert_y_close(y, oracle.dense_linear_ref(x, w), "W = B A")


def test_two_nonzeros_per_group_matches_dense():
    rng = np.random.default_rng(5)
    x = gen.at_most_two_nonzero(rng, 160, 512)
    w = gen.gaussian_bits(rng, (300, 512), 0.02)
    a = gen.gaussian_bits(rng, (16, 512), 0.01)
    b = gen.gaussian_bits(rng, (300, 16), 0.01)
    _, _, scale = rtl.sparsify_2of4(to_dev(x))
    assert (scale.cpu().numpy() == 1.0).all()
    y = y_to_f64(run_sparse_linear(x, w, a, b))
    assert_y_close(y, oracle.dense_linear_ref(x, w), "<= 2 non-zeros")


def test_zero_rows_and_empty_calls():
    rng = np.random.default_rng(6)
    x = gen.mixture_bernoulli(rng, 40, 256)
    x[3] = 0
    x[17] = 0x8000                                     # -0 everywhere
    w = gen.gaussian_bits(rng, (64, 256), 0.02)
    check_sparsify(x)
    y = y_to_f64(run_sparse_linear(x, w, None, None))
    assert (y[3] == 0).all() and (y[17] == 0).all()
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    assert rtl.sparse_linear(empty, to_dev(w)).shape == (0, 64)


def test_subnormal_and_large_magnitude_inputs():
    """Rows of bf16 subnormals (exponent field 0), a row that mixes them with
    normal values, and rows of magnitudes near 1e34 (the fp32 L1 sums stay
    finite): masks bit-exact, scales within 1e-5, the layer within the
    output bar -- over the ordinary and subnormal rows together, and over the
    large rows on their own."""
    rng = np.random.default_rng(43)
    for k in (256, 1024):
        say(f"[parity] subnormal / large magnitudes K={k}")
        x = gen.mixture_bernoulli(rng, 48, k)
        sub = (rng.integers(1, 128, size=(4, k)) | (rng.integers(0, 2, size=(4, k)) << 15)).astype(np.uint16)
        x[0:4] = sub
        x[4] = np.where(rng.random(k) < 0.5, sub[0], x[4])
        x[8:12] = gen.f32_to_bf16_bits(rng.standard_normal((4, k)).astype(np.float32) * np.float32(1e34))
        check_sparsify(x)
        w = gen.gaussian_bits(rng, (200, k), 0.02)
        a = gen.gaussian_bits(rng, (16, k), 0.01)
        b = gen.gaussian_bits(rng, (200, 16), 0.01)
        y = y_to_f64(run_sparse_linear(x, w, a, b))
        ref = oracle.sparse_linear_ref(x, w, a, b)
        big = np.arange(8, 12)
        rest = np.setdiff1d(np.arange(48), big)
        assert_y_close(y[rest], ref[rest], f"ordinary and subnormal rows K={k}")
        assert_y_close(y[big], ref[big], f"rows near 1e34 K={k}")


def test_wrappers_reject_bad_out_and_workspace():
    """An output or workspace the kernels could not write safely is refused
    before any launch, and the valid call afterwards is unaffected."""
    rng = np.random.default_rng(3)
    x = to_dev(gen.mixture_bernoulli(rng, 64, 256))
    w = to_dev(gen.gaussian_bits(rng, (96, 256), 0.02))
    bad_outs = [torch.empty((64, 95), dtype=torch.bfloat16, device=DEV),
                torch.empty((64, 96), dtype=torch.float32, device=DEV),
                torch.empty((96, 64), dtype=torch.bfloat16, device=DEV).t(),
                torch.empty((64, 96), dtype=torch.bfloat16)]
    for o in bad_outs:
        with pytest.raises((TypeError, ValueError)):
            rtl.sparse_linear(x, w, out=o)
        with pytest.raises((TypeError, ValueError)):
            rtl.dense_linear(x, w, out=o)
    need = rtl.sparse_linear_workspace_bytes(64, 256, 0)
    for ws in [torch.empty((need,), dtype=torch.float32, device=DEV),
               torch.empty((need,), dtype=torch.uint8)]:
        with pytest.raises((TypeError, ValueError)):
            rtl.sparse_linear(x, w, workspace=ws)
    y = torch.empty((64, 96), dtype=torch.bfloat16, device=DEV)
    rtl.sparse_linear(x, w, out=y)
    torch.cuda.synchronize()
    xh = to_host(x)
    assert_y_close(y_to_f64(y), oracle.sparse_linear_ref(xh, to_host(w)), "after rejected calls")


def test_bitwise_repeatable():
    x, w, a, b = gen.make_config("attn_proj", m=512)
    y1 = to_host(run_sparse_linear(x, w, a, b))
    y2 = to_host(run_sparse_linear(x, w, a, b))
    assert np.array_equal(y1, y2)


def test_hip_graph_capture_replays():
    """The layer and the prepare / apply pair (per-tensor compensation: three
    kernels in its prepare) captured in a HIP graph on preallocated outputs
    and workspace: every replay, with eager work between replays that
    overwrites the outputs and the workspace, matches the eager call bit for
    bit.  The library's calls allocate, synchronise and clear nothing."""
    x, w, a, b = gen.make_config("attn_proj", m=512)
    m, k = x.shape
    n = w.shape[0]
    xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
    need = rtl.sparse_linear_workspace_bytes(m, k, a.shape[0])
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ws1 = torch.empty((need,), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty((need,), dtype=torch.uint8, device=DEV)

    def calls():
        rtl.sparse_linear(xd, wd, ad, bd, 0.5, out=y1, workspace=ws1)
        rtl.apply(rtl.prepare(xd, ad, 0.5, workspace=ws2, variant=rtl.COMP_TENSOR), wd, bd, out=y2)

    calls()
    torch.cuda.synchronize()
    e1, e2 = to_host(y1), to_host(y2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for i in range(4):
        say(f"[parity] graph replay {i}")
        y1.zero_()
        y2.zero_()
        ws1.fill_(i + 1)
        ws2.fill_(i + 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y1), e1), f"replay {i}: sparse_linear"
        assert np.array_equal(to_host(y2), e2), f"replay {i}: prepare (per tensor) + apply"


def test_concurrent_streams():
    """Two layers launched on two streams at once, each with its own output
    and workspace, give what they give one after the other: the library
    keeps no state between calls."""
    rng = np.random.default_rng(47)
    cases = []
    for m, k, n, r in ((640, 1024, 768, 64), (300, 2048, 520, 32)):
        x = gen.mixture_bernoulli(rng, m, k)
        w = gen.gaussian_bits(rng, (n, k), 0.02)
        a = gen.gaussian_bits(rng, (r, k), 0.01)
        b = gen.gaussian_bits(rng, (n, r), 0.01)
        cases.append(tuple(to_dev(t) for t in (x, w, a, b)))
    seq = [to_host(rtl.sparse_linear(*c)) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = []
    for rep in range(3):
        outs.clear()
        for c, st in zip(cases, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(rtl.sparse_linear(*c))
        torch.cuda.synchronize()
        for got, want in zip(outs, seq):
            assert np.array_equal(to_host(got), want), f"round {rep}"


FULL = ["attn_proj", "mlp_up", "mlp_down", "textimg_p05", "textimg_p10", "textimg_p25",
        "mlp_up_share8", "textimg_share8", "textimg_share2"]


def assert_all_rows_close(y_dev, ref, what, block=1024):
    """Every element of a full-size output against the oracle's, with the
    rms of the whole reference; the device output comes over in row blocks."""
    rms = np.sqrt(np.mean(ref ** 2))
    for i0 in range(0, ref.shape[0], block):
        assert_y_close(y_to_f64(y_dev[i0:i0 + block]), ref[i0:i0 + block], f"{what} rows {i0}+", rms=rms)


@pytest.mark.parametrize("name", FULL)
def test_full_size_config(name):
    """Each full workload: every mask, value and scale, and every element of
    Y from the fused layer and from the dense baseline."""
    cfg = gen.config(name)
    say(f"[parity] full config {name}: M={cfg.m} K={cfg.k} N={cfg.n} r={cfg.r}")
    x, w, a, b = gen.make_config(name)
    check_sparsify(x)
    xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
    y = rtl.sparse_linear(xd, wd, ad, bd)
    yd = rtl.dense_linear(xd, wd)
    torch.cuda.synchronize()
    assert_all_rows_close(y, oracle.sparse_linear_ref(x, w, a, b), f"{name} sparse")
    assert_all_rows_close(yd, oracle.dense_linear_ref(x, w), f"{name} dense")


def test_prepare_once_apply_many():
    """One prepare feeding several weights (projections that share an input)
    gives what separate sparse_linear calls give, bit for bit."""
    rng = np.random.default_rng(31)
    x = gen.mixture_bernoulli(rng, 384, 1024)
    a = gen.gaussian_bits(rng, (64, 1024), 0.01)
    xd, ad = to_dev(x), to_dev(a)
    prep = rtl.prepare(xd, ad, 0.5)
    for n in (256, 520, 1024):
        w = gen.gaussian_bits(rng, (n, 1024), 0.02)
        b = gen.gaussian_bits(rng, (n, 64), 0.01)
        y1 = to_host(rtl.apply(prep, to_dev(w), to_dev(b)))
        y2 = to_host(rtl.sparse_linear(xd, to_dev(w), ad, to_dev(b), lora_scale=0.5))
        assert np.array_equal(y1, y2)
        assert_y_close(oracle.bf16_bits_to_f64(y1), oracle.sparse_linear_ref(x, w, a, b, 0.5), f"apply N={n}")


COMPRESSED_SHAPES = [
    # (M, K, N): K % 16 == 0, == 4, == 8, == 12; ragged M and N; one group; many tiles
    (64, 256, 128), (300, 516, 200), (257, 1000, 333), (1, 4, 1), (5, 12, 7), (33, 260, 300),
    (512, 3072, 520),
]


@pytest.mark.parametrize("shape", COMPRESSED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_compressed_linear_small_and_ragged(shape):
    """rtl_sparse_linear_compressed on the oracle's canonical compressed form,
    with and without the per-token scale."""
    m, k, n = shape
    say(f"[parity] compressed M={m} K={k} N={n}")
    rng = np.random.default_rng(m * 7 + k + n)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    _, _, s, i0, i1 = oracle.sparsify(x)
    vals, idx = oracle.compress(x, i0, i1)
    s32 = s.astype(np.float32)
    vd = to_dev(vals)
    id_ = torch.from_numpy(idx).to(DEV)
    wd = to_dev(w)
    y = rtl.sparse_linear_compressed(vd, id_, torch.from_numpy(s32).to(DEV), wd)
    y0 = rtl.sparse_linear_compressed(vd, id_, None, wd)
    torch.cuda.synchronize()
    assert_y_close(y_to_f64(y), oracle.compressed_linear_ref(vals, idx, s32, w, k), f"compressed {shape}")
    assert_y_close(y_to_f64(y0), oracle.compressed_linear_ref(vals, idx, None, w, k), f"compressed {shape}, no scale")


def test_unfused_sparsify_then_compressed_gemm():
    """The unfused form of the layer without LoRA: rtl_sparsify_2of4 writes
    the canonical compressed X, rtl_sparse_linear_compressed multiplies it;
    the result is the layer (r = 0) within the output bar."""
    for name, m in (("attn_proj", 512), ("mlp_down", 256)):
        x, w, _, _ = gen.make_config(name, m=m, with_lora=False)
        xd = to_dev(x)
        vals, idx, scale = rtl.sparsify_2of4(xd)
        y = rtl.sparse_linear_compressed(vals, idx, scale, to_dev(w))
        torch.cuda.synchronize()
        assert_y_close(y_to_f64(y), oracle.sparse_linear_ref(x, w), f"unfused {name}")


def test_compressed_linear_full_headline():
    cfg = gen.config("mlp_up")
    say(f"[parity] compressed full mlp_up: M={cfg.m} K={cfg.k} N={cfg.n}")
    x, w, _, _ = gen.make_config("mlp_up", with_lora=False)
    vals, idx, scale = rtl.sparsify_2of4(to_dev(x))
    y = rtl.sparse_linear_compressed(vals, idx, scale, to_dev(w))
    torch.cuda.synchronize()
    assert_all_rows_close(y, oracle.sparse_linear_ref(x, w), "compressed full mlp_up")


COMP = {"token": rtl.COMP_TOKEN, "none": rtl.COMP_NONE, "tensor": rtl.COMP_TENSOR, "group": rtl.COMP_GROUP}
LORA = {"residual": rtl.LORA_RESIDUAL, "pruned": rtl.LORA_PRUNED, "input": rtl.LORA_INPUT}
VARIANT_SHAPES = [
    # (M, K, N, r): DMA pre-pass with K % 128 == 0; DMA with a channel tail;
    # the generic pre-pass for r > 64; the generic one for K % 8 == 4; the
    # generic one loading A per k-pair (rank 128, and rank 64 with K % 8 == 4
    # under per-group compensation) over two k-pairs per wavefront
    (256, 1024, 160, 32), (300, 520, 200, 24), (64, 256, 96, 96), (33, 260, 100, 16),
    (200, 2052, 136, 64), (160, 2048, 120, 128),
]


@pytest.mark.parametrize("comp", list(COMP))
@pytest.mark.parametrize("lora", list(LORA))
def test_variants_against_oracle(comp, lora):
    for m, k, n, r in VARIANT_SHAPES:
        say(f"[parity] variant comp={comp} lora={lora} M={m} K={k} N={n} r={r}")
        rng = np.random.default_rng(m + k + n + r)
        x = gen.mixture_bernoulli(rng, m, k)
        w = gen.gaussian_bits(rng, (n, k), 0.02)
        a = gen.gaussian_bits(rng, (r, k), 0.05)
        b = gen.gaussian_bits(rng, (n, r), 0.05)
        prep = rtl.prepare(to_dev(x), to_dev(a), 0.75, variant=COMP[comp] | LORA[lora])
        y = rtl.apply(prep, to_dev(w), to_dev(b))
        torch.cuda.synchronize()
        ref = oracle.sparse_linear_variant_ref(x, w, a, b, 0.75, comp=comp, lora=lora)
        assert_y_close(y_to_f64(y), ref, f"comp={comp} lora={lora} {(m, k, n, r)}")


def test_variant_tensor_and_group_full_headline():
    x, w, a, b = gen.make_config("mlp_up")
    xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
    for comp in ("tensor", "group"):
        say(f"[parity] full mlp_up variant comp={comp}")
        y = rtl.apply(rtl.prepare(xd, ad, 1.0, variant=COMP[comp]), wd, bd)
        torch.cuda.synchronize()
        ref = oracle.sparse_linear_variant_ref(x, w, a, b, 1.0, comp=comp)
        assert_all_rows_close(y, ref, f"full mlp_up comp={comp}")


@pytest.mark.parametrize("shape", [(4103, 520, 12248, 24), (4100, 512, 12250, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ragged_wide_tiles(shape):
    """Large ragged layers (17 row tiles, N not a multiple of 64): these take
    256-column tiles (the 192-column ones would need an extra round of
    tiles), in the channel-tail and the full-K copy modes."""
    m, k, n, r = shape
    say(f"[parity] ragged wide M={m} K={k} N={n} r={r}")
    rng = np.random.default_rng(m + n)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01)
    b = gen.gaussian_bits(rng, (n, r), 0.01)
    y = run_sparse_linear(x, w, a, b)
    assert_all_rows_close(y, oracle.sparse_linear_ref(x, w, a, b), f"ragged wide {shape}")


@pytest.mark.parametrize("shape", [(8000, 520, 3000, 32), (8192, 512, 3072, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_narrow_tiles_several_per_workgroup(shape):
    """192-column tiles with two tiles per persistent workgroup on 256 CUs
    (512 tiles of 256 x 192 against 384 of 256 x 256: two rounds either
    way, so the narrower tile is taken): the cross-tile copy pipeline, the
    staged epilogue and the staggered refills of the 192-column instance,
    in the channel-tail and the full-K copy modes."""
    m, k, n, r = shape
    say(f"[parity] narrow tiles M={m} K={k} N={n} r={r}")
    rng = np.random.default_rng(m + k + n)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01)
    b = gen.gaussian_bits(rng, (n, r), 0.01)
    y = run_sparse_linear(x, w, a, b)
    assert_all_rows_close(y, oracle.sparse_linear_ref(x, w, a, b), f"narrow tiles {shape}")


def _path_cases(count=40, seed=20261204):
    """Seeded random layers over every entry point that computes the layer:
    rtl_sparse_linear, prepare_variant + apply (a random compensation and
    LoRA input), the allocation-free call, and the layer policy with the
    streamed-weights hint; M up to 6000 and N up to 7000 (several tiles per
    persistent workgroup), K a multiple of 4 or of 128, ranks 0 to 128."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        m = int(rng.choice([rng.integers(1, 300), rng.integers(256, 2600), rng.integers(2600, 6000)]))
        k = 4 * int(rng.integers(1, 700)) if rng.random() < 0.7 else 128 * int(rng.integers(1, 20))
        n = int(rng.choice([rng.integers(1, 2500), rng.integers(2500, 7000)]))
        r = int(rng.choice([0, 5, 8, 16, 24, 32, 48, 64, 64, 96, 128]))
        path = str(rng.choice(["layer", "variant", "noalloc", "stream"]))
        comp, lora = str(rng.choice(list(COMP))), str(rng.choice(list(LORA)))
        cases.append((i, m, k, n, r, path, comp, lora))
    return cases


@pytest.mark.parametrize("case", _path_cases(), ids=lambda c: f"{c[0]}-{c[5]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}")
def test_random_entry_point_sweep(case):
    from activation_sparse_gemm_token_amd import layers
    i, m, k, n, r, path, comp, lora = case
    say(f"[parity] path sweep {i}: {path} M={m} K={k} N={n} r={r}" + (f" {comp}/{lora}" if path == "variant" else ""))
    rng = np.random.default_rng(1000 + i)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01) if r else None
    b = gen.gaussian_bits(rng, (n, r), 0.01) if r else None
    xd, wd = to_dev(x), to_dev(w)
    ad, bd = (to_dev(a), to_dev(b)) if r else (None, None)
    alpha = 0.75
    if path == "variant":
        y = rtl.apply(rtl.prepare(xd, ad, alpha, variant=COMP[comp] | LORA[lora]), wd, bd)
        ref = oracle.sparse_linear_variant_ref(x, w, a, b, alpha, comp=comp, lora=lora)
    else:
        if path == "layer":
            y = rtl.sparse_linear(xd, wd, ad, bd, alpha)
        elif path == "noalloc":
            y = rtl.sparse_linear_noalloc(xd, wd, ad, bd, alpha)
        else:
            y = layers.LayerPolicy(1, stream_weights=True).linear(0, xd, wd, ad, bd, alpha)
            plain = rtl.sparse_linear(xd, wd, ad, bd, alpha)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(y), to_host(plain)), "the streamed-weights hint changed the output"
        ref = oracle.sparse_linear_ref(x, w, a, b, alpha)
    torch.cuda.synchronize()
    assert_y_close(y_to_f64(y), ref, f"path sweep {i} ({path})")
