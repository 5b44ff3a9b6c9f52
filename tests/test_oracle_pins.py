"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test states the fact it checks: brute force over tiny inputs, a
hand-worked case, an invariant, a closed form, or a library routine.  The
sources are the RT-Lynx pages (ai-feeds summary 方法; qingkeai article
sections 01-04; neuraltrendhub "What the paper found").  The mutation tests at
the end plant plausible mistakes in a copy of the oracle and check that at
least one pin catches each.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import rtlynx_ref as ref
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_2of4.json")


def _bits(vals):
    return gen.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ---------------------------------------------------------------- selection

def _alphabet_bits():
    # {-3, -2, -1, -0, +0, 1, 2, 3} as bf16 words
    return _bits([-3.0, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0, 3.0])


def test_selection_equals_brute_force_exhaustive_small_alphabet():
    """All 8^4 = 4096 groups over a signed alphabet with both zeros: the rank
    rule keeps exactly the pair that the six-pattern enumeration picks
    (largest kept |x| sum, lexicographically first on ties)."""
    al = _alphabet_bits()
    tuples = np.array(list(itertools.product(range(8), repeat=4)))
    bits = al[tuples].reshape(1, -1)
    mask, i0, i1 = oracle.select_2of4(bits)
    b0, b1 = oracle.brute_force_select_2of4(bits)
    assert np.array_equal(i0, b0) and np.array_equal(i1, b1)
    assert (mask.reshape(-1, 4).sum(axis=1) == 2).all()
    assert (i0 < i1).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_equals_brute_force_random_bf16(seed):
    """Random finite bf16 words over the whole exponent range, subnormals
    included, plus many exact ties (values drawn from a small pool)."""
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 1 << 16, size=(16, 1024), dtype=np.uint32).astype(np.uint16)
    finite = (raw & 0x7F80) != 0x7F80
    raw = np.where(finite, raw, raw & 0x807F)          # turn Inf/NaN into subnormals
    pool = rng.choice(raw.reshape(-1), size=5)
    raw[:, 512:] = pool[rng.integers(0, 5, size=(16, 512))] ^ (rng.integers(0, 2, size=(16, 512)) << 15).astype(np.uint16)
    mask, i0, i1 = oracle.select_2of4(raw)
    b0, b1 = oracle.brute_force_select_2of4(raw)
    assert np.array_equal(i0, b0) and np.array_equal(i1, b1)


def test_selection_is_optimal_among_all_2of4_masks():
    """No other 2:4 mask keeps a larger L1 (so none prunes a smaller one)."""
    rng = np.random.default_rng(5)
    x = gen.mixture_bernoulli(rng, 32, 512)
    v = np.abs(oracle.bf16_bits_to_f64(x)).reshape(32, 128, 4)
    mask, _, _ = oracle.select_2of4(x)
    kept = np.where(mask.reshape(32, 128, 4), v, 0).sum(axis=2)
    for a, b in itertools.combinations(range(4), 2):
        assert (v[:, :, a] + v[:, :, b] <= kept).all()


def test_keys_order_like_magnitude():
    """The 15-bit key orders every finite bf16 word exactly like |x|."""
    words = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = words[(words & 0x7F80) != 0x7F80]
    keys = oracle.magnitude_keys(finite)
    mags = np.abs(oracle.bf16_bits_to_f64(finite))
    o = np.argsort(keys, kind="stable")
    assert (np.diff(mags[o]) >= 0).all()
    assert np.array_equal(keys[o][1:] == keys[o][:-1], mags[o][1:] == mags[o][:-1])


# ------------------------------------------------------------- hand-worked

with open(GOLDEN) as f:
    _G = json.load(f)


@pytest.mark.parametrize("case", _G["selection_cases"], ids=lambda c: c["why"][:40])
def test_handworked_selection(case):
    bits = _bits(case["x"]).reshape(1, -1)
    sx, mask, s, i0, i1 = oracle.sparsify(bits)
    assert [[int(a), int(b)] for a, b in zip(i0[0], i1[0])] == case["kept"]
    assert s[0] == pytest.approx(case["s"], rel=1e-15)
    np.testing.assert_allclose(sx[0], case["sx"], rtol=1e-15, atol=0)
    vals, idx = oracle.compress(bits)
    assert [f"0x{v:04x}" for v in vals[0]] == case["vals"]
    assert [f"0x{v:02x}" for v in idx[0]] == case["idx_bytes"]
    nib = [(idx[0][g // 2] >> (4 * (g % 2))) & 0xF for g in range(len(case["kept"]))]
    assert nib == case["code_nibbles"]


@pytest.mark.parametrize("case", _G["layer_cases"], ids=lambda c: c["why"][:40])
def test_handworked_layer(case):
    x, w, a, b = (_bits(case[k]) for k in ("x", "w", "a", "b"))
    y = oracle.sparse_linear_ref(x, w, a, b, case["alpha"])
    np.testing.assert_allclose(y, case["y"], rtol=1e-14, atol=1e-14)
    y2 = oracle.sparse_linear_gather_ref(x, w, a, b, case["alpha"])
    np.testing.assert_allclose(y2, case["y"], rtol=1e-14, atol=1e-14)


# -------------------------------------------------------------- invariants

def _inputs(name, m=None):
    return gen.make_config(name, m=m)


@pytest.mark.parametrize("law", ["mixture", "gelu", "exact"])
def test_l1_norm_is_restored(law):
    """Norm compensation restores each token's L1 norm (ai-feeds summary,
    核心模块 1; qingkeai article, section 03.1)."""
    rng = np.random.default_rng(11)
    x = {"mixture": lambda: gen.mixture_bernoulli(rng, 128, 768),
         "gelu": lambda: gen.gelu_of_normal(rng, 128, 768),
         "exact": lambda: gen.mixture_exact_count(rng, 128, 768, 0.05)}[law]()
    sx, mask, s, _, _ = oracle.sparsify(x)
    l1x = np.abs(oracle.bf16_bits_to_f64(x)).sum(axis=1)
    np.testing.assert_allclose(np.abs(sx).sum(axis=1), l1x, rtol=1e-12)
    assert (s >= 1.0).all() and (s <= 2.0).all()
    assert (mask.sum(axis=1) == 768 // 2).all()


def test_scale_is_two_when_all_magnitudes_tie():
    """X = +-c everywhere: every group keeps half its mass, so s = 2 exactly."""
    rng = np.random.default_rng(3)
    signs = rng.choice([-1.0, 1.0], size=(16, 64))
    sx, _, s, _, _ = oracle.sparsify(_bits(0.375 * signs))
    assert (s == 2.0).all()


def test_two_nonzeros_per_group_is_identity():
    """Every group has at most two non-zeros: S(X) = X, s = 1 exactly, the
    residual is zero, so the layer equals the dense product X W^T whatever
    the LoRA factors (fp64 NumPy matmul)."""
    rng = np.random.default_rng(7)
    x = gen.at_most_two_nonzero(rng, 48, 256)
    w = gen.gaussian_bits(rng, (96, 256), 0.02)
    a = gen.gaussian_bits(rng, (8, 256), 0.01)
    b = gen.gaussian_bits(rng, (96, 8), 0.01)
    xv = oracle.bf16_bits_to_f64(x)
    sx, mask, s, _, _ = oracle.sparsify(x)
    assert (s == 1.0).all()
    assert np.array_equal(sx, xv)
    assert (mask | (xv == 0)).all()
    y = oracle.sparse_linear_ref(x, w, a, b)
    np.testing.assert_array_equal(y, np.matmul(xv, oracle.bf16_bits_to_f64(w).T))


def test_sign_and_power_of_two_equivariance():
    rng = np.random.default_rng(9)
    x = gen.mixture_bernoulli(rng, 32, 256)
    xv = oracle.bf16_bits_to_f64(x)
    sx, m0, s0, i00, i10 = oracle.sparsify(x)
    for c in (-1.0, 2.0, -0.25, 8.0):
        xc = gen.f32_to_bf16_bits((xv * c).astype(np.float32))
        assert np.array_equal(oracle.bf16_bits_to_f64(xc), xv * c)
        sxc, mc, sc, i0c, i1c = oracle.sparsify(xc)
        assert np.array_equal(mc, m0) and np.array_equal(i0c, i00) and np.array_equal(i1c, i10)
        np.testing.assert_allclose(sc, s0, rtol=1e-15)
        np.testing.assert_allclose(sxc, c * sx, rtol=1e-15, atol=0)


def test_compress_roundtrip():
    rng = np.random.default_rng(13)
    for k in (4, 12, 256, 260):
        x = gen.mixture_bernoulli(rng, 17, k)
        mask, i0, i1 = oracle.select_2of4(x)
        vals, idx = oracle.compress(x)
        assert vals.shape == (17, k // 2) and idx.shape == (17, (k // 4 + 1) // 2)
        back = oracle.decompress(vals, idx, k)
        assert np.array_equal(back, np.where(mask, x, np.uint16(0)))
        if (k // 4) % 2:
            assert (idx[:, -1] >> 4 == 0).all()


def test_gather_form_equals_masked_dense_form():
    """The compressed-operand product (what a sparse GEMM computes) equals a
    dense fp64 GEMM on the masked, scaled X."""
    x, w, a, b = _inputs("tiny")
    y1 = oracle.sparse_linear_ref(x, w, a, b, 0.7)
    y2 = oracle.sparse_linear_gather_ref(x, w, a, b, 0.7)
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12 * np.abs(y1).max())


def test_compressed_linear_handworked():
    """One group: kept values 2 and 3 at channels 1 and 3 (code 1 | 3 << 2),
    scale 1.5, W row (1, 10, 100, 1000): y = 1.5 (2 * 10 + 3 * 1000) = 4530;
    a second token with the pair at channels 0, 2 and no scale factor."""
    vals = gen.f32_to_bf16_bits(np.array([[2.0, 3.0], [5.0, -1.0]], dtype=np.float32))
    idx = np.array([[1 | (3 << 2)], [0 | (2 << 2)]], dtype=np.uint8)
    w = gen.f32_to_bf16_bits(np.array([[1.0, 10.0, 100.0, 1000.0]], dtype=np.float32))
    y = oracle.compressed_linear_ref(vals, idx, np.array([1.5, 1.0]), w, 4)
    assert y.tolist() == [[4530.0], [5.0 * 1.0 - 1.0 * 100.0]]
    y0 = oracle.compressed_linear_ref(vals, idx, None, w, 4)
    assert y0.tolist() == [[3020.0], [-95.0]]


def test_compressed_linear_equals_layer_without_lora():
    """Compressing X and multiplying the compressed form with its scale is
    the layer without the LoRA branch (r = 0), by two independent routes."""
    for name in ("tiny",):
        x, w, _, _ = _inputs(name)
        k = x.shape[1]
        _, _, s, i0, i1 = oracle.sparsify(x)
        vals, idx = oracle.compress(x, i0, i1)
        y1 = oracle.compressed_linear_ref(vals, idx, s, w, k)
        y2 = oracle.sparse_linear_gather_ref(x, w)
        np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12 * np.abs(y2).max())


def _exact_lora_factors(rng, n, k, r):
    a = gen.f32_to_bf16_bits(rng.integers(-1, 2, size=(r, k)).astype(np.float32) * 0.125)
    b = gen.f32_to_bf16_bits(rng.integers(-1, 2, size=(n, r)).astype(np.float32) * 0.125)
    w = oracle.bf16_bits_to_f64(b) @ oracle.bf16_bits_to_f64(a)       # multiples of 2^-6, |w| <= r/64
    wb = gen.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(wb), w)
    return wb, a, b


def test_lora_on_residual_recovers_dense_when_w_equals_ba():
    """W = B A exactly: S(X) W^T + ((X - S(X)) A^T) B^T = X W^T for any mask
    and scale.  Pins the branch's input (the pruned residual including the
    scale), its sign and the operand orientation."""
    rng = np.random.default_rng(21)
    for name, m in (("tiny", None), ("mlp_down", 16)):
        cfg = gen.config(name)
        x = gen.make_config(name, m=m)[0]
        w, a, b = _exact_lora_factors(rng, 64, cfg.k, 8)
        y = oracle.sparse_linear_ref(x, w, a, b, 1.0)
        yd = oracle.dense_linear_ref(x, w)
        np.testing.assert_allclose(y, yd, rtol=1e-11, atol=1e-11 * np.abs(yd).max())


def test_row_permutation_equivariance():
    x, w, a, b = _inputs("tiny")
    perm = np.random.default_rng(2).permutation(x.shape[0])
    y = oracle.sparse_linear_ref(x, w, a, b)
    yp = oracle.sparse_linear_ref(x[perm], w, a, b)
    np.testing.assert_array_equal(yp, y[perm])


def test_zero_weight_leaves_lora_term():
    x, w, a, b = _inputs("tiny")
    wz = np.zeros_like(w)
    y = oracle.sparse_linear_ref(x, wz, a, b, 2.0)
    t = oracle.lora_down_ref(x, a)
    np.testing.assert_allclose(y, 2.0 * t @ oracle.bf16_bits_to_f64(b).T, rtol=1e-13)
    # R = (1 - M) X + (1 - s) M X: the two 2:4-sparse parts add up to the residual
    sx, mask, s, _, _ = oracle.sparsify(x)
    xv = oracle.bf16_bits_to_f64(x)
    r2 = np.where(mask, 0, xv) + (1 - s)[:, None] * np.where(mask, xv, 0)
    np.testing.assert_allclose(xv - sx, r2, rtol=1e-13, atol=1e-15)


def test_config_shapes():
    for name, cfg in gen.CONFIGS.items():
        assert cfg.k % 4 == 0
    x, w, a, b = _inputs("tiny")
    assert x.shape == (64, 256) and w.shape == (128, 256) and a.shape == (8, 256) and b.shape == (128, 8)


# ------------------------------------------------------------- mutations
# Plausible mistakes planted in a copy of the oracle on the CPU: each must be
# caught by at least one of the independent pins above.

def _pins_pass(mod):
    """Run a subset of the pins against a (possibly mutated) oracle module."""
    al = _alphabet_bits()
    tuples = np.array(list(itertools.product(range(8), repeat=4)))
    bits = al[tuples].reshape(1, -1)
    _, i0, i1 = mod.select_2of4(bits)
    b0, b1 = ref.brute_force_select_2of4(bits)
    if not (np.array_equal(i0, b0) and np.array_equal(i1, b1)):
        return False
    rng = np.random.default_rng(11)
    x = gen.mixture_bernoulli(rng, 64, 256)
    sx = mod.sparsify(x)[0]
    if not np.allclose(np.abs(sx).sum(1), np.abs(ref.bf16_bits_to_f64(x)).sum(1), rtol=1e-12):
        return False
    w, a, b = _exact_lora_factors(np.random.default_rng(1), 32, 256, 8)
    y = mod.sparse_linear_ref(x, w, a, b, 1.0)
    yd = ref.dense_linear_ref(x, w)
    if not np.allclose(y, yd, rtol=1e-11, atol=1e-11 * np.abs(yd).max()):
        return False
    for case in _G["layer_cases"]:
        xs, ws, as_, bs = (_bits(case[k]) for k in ("x", "w", "a", "b"))
        if not np.allclose(mod.sparse_linear_ref(xs, ws, as_, bs, case["alpha"]), case["y"], rtol=1e-12):
            return False
    return True


def _mutant(patch):
    import types
    m = types.ModuleType("mutant")
    m.__dict__.update({k: v for k, v in ref.__dict__.items() if not k.startswith("__")})
    patch(m)
    for fn in ("sparsify", "sparse_linear_ref", "lora_down_ref", "select_2of4"):
        f = m.__dict__[fn]
        if f is getattr(ref, fn):          # untouched: rebind so it calls the mutant's helpers
            m.__dict__[fn] = types.FunctionType(f.__code__, m.__dict__, f.__name__, f.__defaults__)
    return m


def _tie_to_higher(m):
    orig = ref.select_2of4

    def sel(bits):
        b = np.asarray(bits)[:, ::-1]
        mask, i0, i1 = orig(b)
        mask = mask[:, ::-1]
        i0r = (3 - i1[:, ::-1]).astype(np.uint8)
        i1r = (3 - i0[:, ::-1]).astype(np.uint8)
        return mask, i0r, i1r
    m.select_2of4 = sel


def _inverted_scale(m):
    m.compensation_scale = lambda lk, lp: np.where(np.asarray(lk) > 0, np.asarray(lk) / np.maximum(np.asarray(lk) + np.asarray(lp), 1e-300), 1.0)


def _no_scale(m):
    m.compensation_scale = lambda lk, lp: np.ones_like(np.asarray(lk, dtype=np.float64))


def _lora_on_pruned_only(m):
    def lora_down(x_bits, a_bits):
        x = ref.bf16_bits_to_f64(x_bits)
        mask = ref.select_2of4(x_bits)[0]
        return np.where(mask, 0.0, x) @ ref.bf16_bits_to_f64(a_bits).T

    def sl(x_bits, w_bits, a_bits=None, b_bits=None, alpha=1.0):
        sx = m.sparsify(x_bits)[0]
        y = sx @ ref.bf16_bits_to_f64(w_bits).T
        return y + alpha * (lora_down(x_bits, a_bits) @ ref.bf16_bits_to_f64(b_bits).T)
    m.sparse_linear_ref = sl


def _lora_sign_flip(m):
    def sl(x_bits, w_bits, a_bits=None, b_bits=None, alpha=1.0):
        x = ref.bf16_bits_to_f64(x_bits)
        sx = m.sparsify(x_bits)[0]
        y = sx @ ref.bf16_bits_to_f64(w_bits).T
        t = (sx - x) @ ref.bf16_bits_to_f64(a_bits).T
        return y + alpha * (t @ ref.bf16_bits_to_f64(b_bits).T)
    m.sparse_linear_ref = sl


def _keep_smallest(m):
    def sel(bits):
        flipped = (np.uint16(0x7FFF) - (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF))).astype(np.uint16)
        return ref.select_2of4(flipped)
    m.select_2of4 = sel


def test_unmutated_oracle_passes_pin_subset():
    assert _pins_pass(ref)


@pytest.mark.parametrize("mutation", [_tie_to_higher, _inverted_scale, _no_scale,
                                      _lora_on_pruned_only, _lora_sign_flip, _keep_smallest])
def test_planted_mistake_is_caught(mutation):
    assert not _pins_pass(_mutant(mutation))


# ---------------------------------------------------------------------------
# Compensation and LoRA-input variants.

def test_round_to_bf16_handworked_and_nearest():
    r = oracle.round_to_bf16
    assert r(1.0 + 2.0 ** -8) == 1.0                    # tie: to even
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6    # tie: to even (upwards)
    assert r(1.0 + 3 * 2.0 ** -9) == 1.0 + 2.0 ** -7
    assert r(-3.0) == -3.0 and r(0.0) == 0.0
    assert r(0.1) == 0.10009765625
    rng = np.random.default_rng(3)
    v = rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000)
    q = r(v)
    # a bf16 value: the fp32 pattern has zero low half ...
    assert (np.float32(q).view(np.uint32) & 0xFFFF == 0).all()
    # ... and no bf16 neighbour is closer
    bits = np.float32(q).view(np.uint32) >> 16
    for d in (-1, 1):
        nb = ((bits.astype(np.int64) + d).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert (np.abs(q - v) <= np.abs(nb - v)).all()


def test_variant_default_is_the_layer():
    x, w, a, b = _inputs("tiny")
    np.testing.assert_allclose(oracle.sparse_linear_variant_ref(x, w, a, b, 0.7),
                               oracle.sparse_linear_ref(x, w, a, b, 0.7), rtol=1e-13, atol=1e-13)


def test_variant_none_pruned_recovers_dense_when_w_equals_ba():
    """No compensation and the pruned values as the LoRA input: with W = B A
    exactly, (M*X) W^T + ((1-M)*X) A^T B^T = X W^T."""
    rng = np.random.default_rng(21)
    w, a, b = _exact_lora_factors(rng, 24, 64, 8)
    x = gen.mixture_bernoulli(rng, 12, 64)
    y = oracle.sparse_linear_variant_ref(x, w, a, b, 1.0, comp="none", lora="pruned")
    np.testing.assert_allclose(y, oracle.dense_linear_ref(x, w), rtol=1e-12, atol=1e-12)


def test_variant_input_lora_with_zero_weight_is_plain_lora():
    rng = np.random.default_rng(22)
    x = gen.mixture_bernoulli(rng, 9, 32)
    a = gen.gaussian_bits(rng, (4, 32), 0.1)
    b = gen.gaussian_bits(rng, (5, 4), 0.1)
    w = np.zeros((5, 32), dtype=np.uint16)
    f = oracle.bf16_bits_to_f64
    for comp in ("token", "none", "tensor", "group"):
        y = oracle.sparse_linear_variant_ref(x, w, a, b, 0.5, comp=comp, lora="input")
        np.testing.assert_allclose(y, 0.5 * (f(x) @ f(a).T) @ f(b).T, rtol=1e-12, atol=1e-15)


def test_variant_tensor_scale_restores_the_tensor_l1():
    rng = np.random.default_rng(23)
    x = gen.mixture_bernoulli(rng, 10, 64)
    sx, mask = oracle.sparsify_variant(x, "tensor")
    xf = oracle.bf16_bits_to_f64(x)
    np.testing.assert_allclose(np.abs(sx).sum(), np.abs(xf).sum(), rtol=1e-13)
    # one token, or identical tokens: the tensor factor is the token factor
    for xx in (x[:1], np.repeat(x[:1], 5, axis=0)):
        np.testing.assert_allclose(oracle.sparsify_variant(xx, "tensor")[0],
                                   oracle.sparsify_variant(xx, "token")[0], rtol=1e-14)
    # the none variant keeps the values
    sn, mn = oracle.sparsify_variant(x, "none")
    assert np.array_equal(sn, np.where(mn, xf, 0.0))


def test_variant_group_scale_restores_each_group_within_rounding():
    rng = np.random.default_rng(24)
    x = gen.mixture_bernoulli(rng, 16, 128)
    sx, mask = oracle.sparsify_variant(x, "group")
    xf = oracle.bf16_bits_to_f64(x)
    g_s = np.abs(sx).reshape(16, 32, 4).sum(axis=2)
    g_x = np.abs(xf).reshape(16, 32, 4).sum(axis=2)
    # each kept value is s_g x rounded to bf16: within 2^-9 relative each
    assert (np.abs(g_s - g_x) <= 2.0 ** -8 * g_x + 1e-300).all()
    # values are bf16 and kept positions only
    assert (np.float32(sx).view(np.uint32) & 0xFFFF == 0).all()
    assert (sx[~mask] == 0).all()
    # at most two non-zeros per group: S(X) = X exactly
    x2 = gen.at_most_two_nonzero(rng, 8, 64)
    assert np.array_equal(oracle.sparsify_variant(x2, "group")[0], oracle.bf16_bits_to_f64(x2))


def _rne8_exact(q):
    """Round an exact positive rational to 8 significant bits, ties to even,
    in exact arithmetic (brute force: scale into [128, 256) by powers of 2)."""
    from fractions import Fraction
    e = 0
    while q >= 256:
        q /= 2
        e += 1
    while q < 128:
        q *= 2
        e -= 1
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return Fraction(n) * Fraction(2) ** e


def _near_tie_groups(rng, n=1 << 20, rows=16):
    """Groups whose folded values lie on or within 2^-20 (relative) of a bf16
    rounding tie, found among random groups of 8-bit integers: the values
    where the order of the roundings decides the result.  Packed as a
    [rows, ...] bf16 array of whole groups."""
    v = (rng.integers(1, 256, size=(n, 4)) * rng.choice([-1, 1], size=(n, 4))).astype(np.float32) / 64
    bits = gen.f32_to_bf16_bits(v)
    xf = oracle.bf16_bits_to_f64(bits)
    mask, _, _ = oracle.select_2of4(bits)
    ax = np.abs(xf)
    lk = np.where(mask, ax, 0.0).sum(axis=1, keepdims=True)
    tot = ax.sum(axis=1, keepdims=True)
    f, _ = np.frexp(ax * tot / lk)
    t = f * 256.0                                      # in [128, 256): ties at half-integers
    near = (np.abs(t - np.floor(t) - 0.5) < 2.0 ** -12) & mask
    sel = bits[near.any(axis=1)]
    sel = sel[: (len(sel) // rows) * rows]
    assert len(sel) >= 4 * rows
    return sel.reshape(rows, -1)


def test_variant_group_values_are_the_exactly_rounded_products():
    """Every folded value is x (L1 of the group) / (L1 of the kept pair) as an
    exact rational, rounded once to bf16 with ties to even: checked in exact
    arithmetic, on random mixtures and on small integers, where products land
    on bf16 ties and near them."""
    from fractions import Fraction
    rng = np.random.default_rng(25)
    cases = [gen.mixture_bernoulli(rng, 6, 64),
             gen.f32_to_bf16_bits(rng.integers(-300, 301, size=(8, 64)).astype(np.float32)),
             gen.f32_to_bf16_bits((rng.integers(1, 256, size=(8, 64)) * rng.choice([-1, 1], (8, 64)))
                                  .astype(np.float32) / 64),
             _near_tie_groups(rng)]
    for x in cases:
        sx, mask = oracle.sparsify_variant(x, "group")
        xf = oracle.bf16_bits_to_f64(x)
        m, k = x.shape
        for i in range(m):
            for g in range(k // 4):
                vals = [Fraction(float(v)) for v in xf[i, 4 * g:4 * g + 4]]
                kept = [j for j in range(4) if mask[i, 4 * g + j]]
                lk = sum(abs(vals[j]) for j in kept)
                tot = sum(abs(v) for v in vals)
                for j in range(4):
                    got = Fraction(float(sx[i, 4 * g + j]))
                    if j not in kept or vals[j] == 0:
                        assert got == 0
                        continue
                    q = abs(vals[j]) * tot / lk
                    want = _rne8_exact(q) * (1 if vals[j] > 0 else -1)
                    assert got == want, (i, g, j, float(got), float(want))
