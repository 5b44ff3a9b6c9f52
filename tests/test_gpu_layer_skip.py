"""Selective layer skipping on the GPU: under a layer policy, skipped
layers give exactly what rtl_dense_linear gives and sparse layers exactly
what rtl_sparse_linear (or the variant's prepare + apply) gives, bit for bit;
a skipped layer is the oracle's dense product; and the streamed-weights hint
(the GEMM instance that probes W into L2) changes no output bit."""
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
from activation_sparse_gemm_token_amd import layers  # noqa: E402

DEV = "cuda:0"


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_policy_dispatch_is_bit_exact():
    rng = np.random.default_rng(77)
    variant = rtl.COMP_NONE | rtl.LORA_PRUNED
    policy = layers.LayerPolicy(5, dense=(1, 3), variants={2: variant})
    shapes = [(300, 1024, 520, 64), (257, 3072, 768, 64), (128, 520, 300, 32), (64, 1028, 200, 16),
              (512, 2048, 1024, 64)]
    for layer, (m, k, n, r) in enumerate(shapes):
        print(f"[layer-skip] layer {layer} mode {policy.mode(layer):#x} M={m} K={k} N={n} r={r}",
              file=sys.stderr, flush=True)
        x = gen.mixture_bernoulli(rng, m, k)
        w = gen.gaussian_bits(rng, (n, k), 0.02)
        a = gen.gaussian_bits(rng, (r, k), 0.01)
        b = gen.gaussian_bits(rng, (n, r), 0.01)
        xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
        got = to_host(policy.linear(layer, xd, wd, ad, bd, 0.5))
        mode = policy.mode(layer)
        if mode == layers.DENSE:
            want = to_host(rtl.dense_linear(xd, wd))
            y = oracle.bf16_bits_to_f64(got)
            ref = oracle.dense_linear_ref(x, w)
            tol = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
            assert (np.abs(y - ref) <= tol).all(), f"layer {layer}: dense product out of tolerance"
        elif mode == 0:
            want = to_host(rtl.sparse_linear(xd, wd, ad, bd, 0.5))
        else:
            want = to_host(rtl.apply(rtl.prepare(xd, ad, 0.5, variant=mode), wd, bd))
        torch.cuda.synchronize()
        assert np.array_equal(got, want), f"layer {layer} (mode {mode:#x}) differs from its entry point"


@pytest.mark.parametrize("shape", [(300, 1024, 520, 64), (4096, 3072, 12288, 64), (1152, 3072, 3072, 64),
                                   (257, 1032, 768, 32), (64, 1028, 200, 16), (200, 2048, 1000, 8),
                                   (8000, 520, 3000, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_streamed_weights_hint_changes_no_bit(shape):
    """The probing GEMM instance (256- and 192-column tiles, one or several
    per workgroup, K % 128 == 0 and only K % 8 == 0, ragged N) against the
    default one: identical outputs; a shape outside the ring (r % 8 != 0,
    K % 8 == 4) ignores the hint."""
    m, k, n, r = shape
    print(f"[layer-skip] streamed weights M={m} K={k} N={n} r={r}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(m + k + n + r)
    x = gen.mixture_bernoulli(rng, m, k)
    w = gen.gaussian_bits(rng, (n, k), 0.02)
    a = gen.gaussian_bits(rng, (r, k), 0.01)
    b = gen.gaussian_bits(rng, (n, r), 0.01)
    xd, wd, ad, bd = to_dev(x), to_dev(w), to_dev(a), to_dev(b)
    variant = rtl.COMP_GROUP | rtl.LORA_PRUNED
    plain = layers.LayerPolicy(2, variants={1: variant})
    streamed = layers.LayerPolicy(2, variants={1: variant}, stream_weights=True)
    outs = []
    for layer in (0, 1):
        want = to_host(plain.linear(layer, xd, wd, ad, bd, 0.75))
        got = to_host(streamed.linear(layer, xd, wd, ad, bd, 0.75))
        torch.cuda.synchronize()
        assert np.array_equal(got, want), f"layer {layer}: the streamed-weights GEMM changed the output"
        outs.append(got)
    if m <= 512:
        # the streamed default layer against the oracle, every element
        ref = oracle.sparse_linear_ref(x, w, a, b, 0.75)
        y = oracle.bf16_bits_to_f64(outs[0])
        tol = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
        assert (np.abs(y - ref) <= tol).all(), "streamed default layer out of tolerance"
