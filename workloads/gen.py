"""Seeded synthetic inputs for the 2:4 activation-sparse linear layer.

This module only draws numbers.  It holds none of the layer's arithmetic: no
selection, no scale, no product.  Both the CPU oracle's tests and the GPU
tests/bench take their inputs from here, as raw bf16 bit patterns
(``numpy.uint16``), so the two sides always see identical bits.

Shapes and laws follow the DiT linear layers that the RT-Lynx pages measure
on (RT-Lynx, qingkeai article sections 02 and 05; neuraltrendhub summary
"What the paper found"):

* token-wise activations are sparse, only about 5-10 % of channels active per
  token: modelled as a two-component mixture, "large" N(0, 4^2) and
  "small" N(0, 0.05^2);
* weights are roughly Gaussian with a wide non-zero spread: N(0, 0.02^2);
* LoRA rank 64, factors N(0, 0.01^2);
* post-GELU activations for the MLP down-projection: GELU(z), z ~ N(-1, 1).

The public datasets and model weights the pages use are not available; these
draws stand in for them.

Every draw is made in float32 (GELU in float64, then float32) and rounded to
bf16 with round-to-nearest-even.  Independent streams for X, W, A and B come
from ``numpy.random.SeedSequence(seed).spawn(4)``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
from scipy.special import erf

__all__ = [
    "Config", "CONFIGS", "config", "make_config", "f32_to_bf16_bits",
    "mixture_bernoulli", "mixture_exact_count", "gelu_of_normal",
    "gaussian_bits", "tie_heavy", "at_most_two_nonzero", "uniform_bits",
]


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the upper 16 bits as uint16.  Inputs are finite by construction.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def _rngs(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4)]


def mixture_bernoulli(rng, m: int, k: int, p: float = 0.08,
                      big: float = 4.0, small: float = 0.05) -> np.ndarray:
    """Each element independently: with probability p ~ N(0, big^2), else N(0, small^2)."""
    z = rng.standard_normal((m, k), dtype=np.float32)
    hot = rng.random((m, k), dtype=np.float32) < np.float32(p)
    z *= np.where(hot, np.float32(big), np.float32(small))
    return f32_to_bf16_bits(z)


def mixture_exact_count(rng, m: int, k: int, p: float,
                        big: float = 4.0, small: float = 0.05) -> np.ndarray:
    """Exactly round(p*k) large channels per token, support drawn uniformly
    without replacement, independently per token; the rest small."""
    n_big = int(round(p * k))
    z = rng.standard_normal((m, k), dtype=np.float32)
    z *= np.float32(small)
    if n_big > 0:
        keys = rng.random((m, k), dtype=np.float32)
        cols = np.argpartition(keys, n_big - 1, axis=1)[:, :n_big]
        rows = np.arange(m)[:, None]
        z[rows, cols] = rng.standard_normal((m, n_big), dtype=np.float32) * np.float32(big)
    return f32_to_bf16_bits(z)


def gelu_of_normal(rng, m: int, k: int, mean: float = -1.0, std: float = 1.0) -> np.ndarray:
    """GELU (exact erf form) of N(mean, std^2) pre-activations."""
    z = rng.standard_normal((m, k)) * std + mean
    g = 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    return f32_to_bf16_bits(g.astype(np.float32))


def gaussian_bits(rng, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def tie_heavy(rng, m: int, k: int) -> np.ndarray:
    """Values from {0, +-1, +-2, +-4} (and -0): most groups hold equal magnitudes."""
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], dtype=np.float32)
    return f32_to_bf16_bits(alphabet[rng.integers(0, alphabet.size, size=(m, k))])


def at_most_two_nonzero(rng, m: int, k: int) -> np.ndarray:
    """Every group of 4 consecutive channels holds at most two non-zeros."""
    z = rng.standard_normal((m, k // 4, 4), dtype=np.float32)
    n_nz = rng.integers(0, 3, size=(m, k // 4, 1))
    slot = np.argsort(np.argsort(rng.random((m, k // 4, 4)), axis=2), axis=2)
    z[slot >= n_nz] = 0.0
    return f32_to_bf16_bits(z.reshape(m, k))


def uniform_bits(rng, shape, emax: int = 0, span: int = 6) -> np.ndarray:
    """bf16 bit patterns drawn directly, for tensors of a billion elements:
    random sign and 7-bit mantissa, exponent uniform over the `span`
    binades below 2^emax (magnitudes in [2^(emax - span), 2^emax)).  Fast
    (integer draws only), so the largest tensors the interface admits can
    be made in seconds."""
    shape = tuple(int(v) for v in np.atleast_1d(shape))
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    exp = (np.uint16(127 + emax - span) + (bits >> np.uint16(7)) % np.uint16(span)).astype(np.uint16)
    sign_mant = rng.integers(0, 1 << 8, size=shape, dtype=np.uint16)
    return (((sign_mant & np.uint16(0x80)) << np.uint16(8)) | (exp << np.uint16(7))
            | (sign_mant & np.uint16(0x7F))).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    m: int
    k: int
    n: int
    r: int
    x_law: str          # "mixture", "gelu", "exact"
    p: float            # active fraction (mixture / exact)
    seed: int
    note: str = ""

    @property
    def flops_dense(self) -> int:
        return 2 * self.m * self.n * self.k


CONFIGS = {
    "tiny": Config("tiny", 64, 256, 128, 8, "mixture", 0.08, 1,
                   "parity-only tiny layer"),
    "attn_proj": Config("attn_proj", 4096, 3072, 3072, 64, "mixture", 0.08, 2,
                        "DiT attention projection, 64x64 latent patches"),
    "mlp_up": Config("mlp_up", 4096, 3072, 12288, 64, "mixture", 0.08, 3,
                     "DiT MLP up-projection (headline shape)"),
    "mlp_down": Config("mlp_down", 4096, 12288, 3072, 64, "gelu", 0.0, 4,
                       "DiT MLP down-projection on post-GELU activations"),
    "textimg_p05": Config("textimg_p05", 9216, 3072, 12288, 64, "exact", 0.05, 5,
                          "2 x (4096 image + 512 text) tokens, 5% active"),
    "textimg_p10": Config("textimg_p10", 9216, 3072, 12288, 64, "exact", 0.10, 6,
                          "2 x (4096 image + 512 text) tokens, 10% active"),
    "textimg_p25": Config("textimg_p25", 9216, 3072, 12288, 64, "exact", 0.25, 7,
                          "2 x (4096 image + 512 text) tokens, 25% active"),
    # One GPU's share of a token-sharded layer (every token is independent,
    # so a share is just a shorter call): the MLP up-projection over 8 GPUs,
    # the text+image batch over 8 and over 2 GPUs (one image + text stream).
    "mlp_up_share8": Config("mlp_up_share8", 512, 3072, 12288, 64, "mixture", 0.08, 8,
                            "DiT MLP up-projection, one of 8 token shards"),
    "textimg_share8": Config("textimg_share8", 1152, 3072, 12288, 64, "exact", 0.05, 9,
                             "text+image batch, one of 8 token shards, 5% active"),
    "textimg_share2": Config("textimg_share2", 4608, 3072, 12288, 64, "exact", 0.05, 10,
                             "text+image batch, one of 2 token shards (4096 image + 512 text), 5% active"),
}


def config(name: str) -> Config:
    return CONFIGS[name]


def make_config(cfg, m: int | None = None, with_lora: bool = True):
    """Draw (x, w, a, b) bf16 bit arrays for ``cfg`` (a Config or its name).

    ``m`` optionally truncates the token count (the first ``m`` rows of the
    full draw are *not* reproduced; a smaller draw is made from the same
    seed, which is what parity tests at reduced size need).
    Returns x[M,K], w[N,K], a[r,K], b[N,r] as uint16 (a, b are None if r == 0
    or ``with_lora`` is False).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    m = cfg.m if m is None else m
    rx, rw, ra, rb = _rngs(cfg.seed)
    if cfg.x_law == "mixture":
        x = mixture_bernoulli(rx, m, cfg.k, cfg.p)
    elif cfg.x_law == "gelu":
        x = gelu_of_normal(rx, m, cfg.k)
    elif cfg.x_law == "exact":
        x = mixture_exact_count(rx, m, cfg.k, cfg.p)
    else:
        raise ValueError(cfg.x_law)
    w = gaussian_bits(rw, (cfg.n, cfg.k), 0.02)
    if with_lora and cfg.r > 0:
        a = gaussian_bits(ra, (cfg.r, cfg.k), 0.01)
        b = gaussian_bits(rb, (cfg.n, cfg.r), 0.01)
    else:
        a = b = None
    return x, w, a, b
