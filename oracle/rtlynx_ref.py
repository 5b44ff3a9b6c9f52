"""Plain fp64 reference of the online 2:4 activation-sparse linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): not part of the
product path, never imported by it.

Sources, cited by page and section:

* ai-feeds summary "RT-Lynx：为扩散模型正确应用GEMM稀疏性", section 方法 /
  输入与稀疏化策略: the input is a DiT linear layer's activation [B, N, C];
  a 2:4 pattern (keep 2 of every 4 values) is applied to it at inference.
* same page, 方法 / 核心模块 1 (norm-compensated sparsification): the L1 norm
  of the pruned elements is redistributed proportionally onto the kept
  activations.
* qingkeai article "RT-Lynx", section 01: each 4 consecutive elements keep
  only 2 non-zeros; section 02: the layer becomes Y = S(X) W^T with S(X) the
  runtime 2:4-sparse activation and W the dense frozen weight; section 03.1:
  Top-K lowers the activation magnitude, which norm compensation restores by
  rescaling; section 03.2: a LoRA branch restores the pruned fine-grained
  residual, backbone frozen; section 04: the fused path covers the 2:4
  pattern decision, Top-K, compression, layout generation, sparse GEMM and
  the LoRA residual.
* neuraltrendhub summary, "What the paper found": LoRA rank 64.

Readings where the pages leave a step open:

* "Top-K" / "keep 2 of 4" ranks by magnitude |x|; ties go to the lower
  channel index, which makes the kept set unique.
* a group is 4 consecutive input channels of one token.
* compensation is per token and multiplicative:
  s = (L1 kept + L1 pruned) / L1 kept, applied to the kept values with their
  signs; s = 1 for an all-zero token.
* the LoRA branch acts on the pruned residual R = X - S(X):
  Y = S(X) W^T + alpha * (R A^T) B^T, with A [r, K], B [N, r].

Data are bf16 bit patterns (numpy uint16); every computation below decodes
them exactly to float64.
"""
from __future__ import annotations

import itertools

import numpy as np

_PAIRS = tuple(itertools.combinations(range(4), 2))   # the 6 keep-patterns of a group


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns: the bf16 word is the top half of
    an IEEE binary32, so shifting it up and reinterpreting is exact."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def magnitude_keys(bits) -> np.ndarray:
    """|x| ordering key: a bf16 word with its sign bit cleared.

    For finite values the unsigned 15-bit pattern is monotone in |x| (sign and
    magnitude format, exponent above mantissa), and -0 and +0 share key 0.
    """
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.int32)


def select_2of4(bits):
    """Top-2 of every group of 4 consecutive channels, by magnitude.

    (ai-feeds summary, 输入与稀疏化策略; qingkeai article, sections 01 and 03.1)

    Element i of a group is outranked by every j with a larger key and by
    every lower-indexed j with an equal key; it is kept iff fewer than two
    elements outrank it.  Exactly two are kept in every group.

    Returns (mask [M, K] bool, idx0 [M, K/4], idx1 [M, K/4]) with idx0 < idx1
    the in-group positions of the kept pair.
    """
    keys = magnitude_keys(bits)
    m, k = keys.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    g = keys.reshape(m, k // 4, 4)
    ki = g[:, :, :, None]       # element i
    kj = g[:, :, None, :]       # element j
    lower = np.tril(np.ones((4, 4), dtype=bool), -1)   # lower[i, j]: j < i
    outranks = (kj > ki) | ((kj == ki) & lower)
    rank = outranks.sum(axis=3)
    keep = rank < 2
    pos = np.arange(4)
    idx0 = np.where(keep, pos, 4).min(axis=2)
    idx1 = np.where(keep, pos, -1).max(axis=2)
    return keep.reshape(m, k), idx0.astype(np.uint8), idx1.astype(np.uint8)


def exact_magnitudes(bits) -> np.ndarray:
    """|x| of bf16 words as exact Python integers in units of 2^-133 (the
    smallest subnormal), so that sums of magnitudes never round."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    e = (b >> 7) & 0xFF
    man = b & 0x7F
    out = np.empty(b.shape, dtype=object)
    flat_e, flat_m, flat_o = e.reshape(-1), man.reshape(-1), out.reshape(-1)
    for i in range(flat_e.size):
        ei, mi = int(flat_e[i]), int(flat_m[i])
        flat_o[i] = mi if ei == 0 else (mi | 0x80) << (ei - 1)
    return out


def brute_force_select_2of4(bits) -> tuple[np.ndarray, np.ndarray]:
    """Independent twin of ``select_2of4`` by enumeration of the six 2:4
    keep-patterns of each group: the pattern whose kept |x| sum is largest,
    summed exactly in integers; among equal sums the lexicographically
    smallest (a, b).  Finite inputs; meant for small arrays."""
    v = exact_magnitudes(bits)
    m, k = v.shape
    g = v.reshape(m, k // 4, 4)
    best = np.full(g.shape[:2], -1, dtype=object)
    bi0 = np.zeros(g.shape[:2], dtype=np.uint8)
    bi1 = np.zeros(g.shape[:2], dtype=np.uint8)
    for a, b in _PAIRS:                       # lexicographic order
        tot = g[:, :, a] + g[:, :, b]
        better = (tot > best).astype(bool)    # strict: earlier pair wins ties
        best = np.where(better, tot, best)
        bi0 = np.where(better, a, bi0).astype(np.uint8)
        bi1 = np.where(better, b, bi1).astype(np.uint8)
    return bi0, bi1


def l1_stats(x: np.ndarray, mask: np.ndarray):
    """Per-token L1 norm of the kept and of the pruned channels (fp64).

    (ai-feeds summary, 核心模块 1: the pruned elements' L1 norm is measured)
    """
    ax = np.abs(x)
    lk = np.where(mask, ax, 0.0).sum(axis=1)
    lp = np.where(mask, 0.0, ax).sum(axis=1)
    return lk, lp


def compensation_scale(lk: np.ndarray, lp: np.ndarray) -> np.ndarray:
    """Per-token factor that redistributes the pruned L1 mass onto the kept
    values in proportion to their own magnitude, restoring the token's L1:
    s = (Lk + Lp) / Lk, and 1 for a token whose kept mass is zero (then the
    whole token is zero).

    (ai-feeds summary, 核心模块 1; qingkeai article, section 03.1)
    """
    lk = np.asarray(lk, dtype=np.float64)
    lp = np.asarray(lp, dtype=np.float64)
    out = np.ones_like(lk)
    nz = lk > 0
    out[nz] = (lk[nz] + lp[nz]) / lk[nz]
    return out


def sparsify(bits):
    """S(X): 2:4 selection plus norm compensation, in fp64, unrounded.

    Returns (S [M, K] fp64, mask, s [M], idx0, idx1).
    """
    x = bf16_bits_to_f64(bits)
    mask, idx0, idx1 = select_2of4(bits)
    lk, lp = l1_stats(x, mask)
    s = compensation_scale(lk, lp)
    sx = np.where(mask, x * s[:, None], 0.0)
    return sx, mask, s, idx0, idx1


def compress(bits, idx0=None, idx1=None):
    """Compressed 2:4 activation: the kept bf16 words, copied bit-exactly and
    unscaled, in index order, plus a 4-bit code idx0 | idx1 << 2 per group.

    (qingkeai article, section 04: activation compression)

    Layout (the library's canonical format): vals [M, K/2] uint16 with group
    g's pair at columns 2g, 2g+1; idx [M, ceil(K/8)] uint8 with group g's code
    in byte g // 2, low nibble for even g, high nibble for odd g, and a zero
    high nibble in the last byte when K/4 is odd.
    """
    b = np.asarray(bits, dtype=np.uint16)
    m, k = b.shape
    if idx0 is None:
        _, idx0, idx1 = select_2of4(b)
    grp = b.reshape(m, k // 4, 4)
    v0 = np.take_along_axis(grp, idx0[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    v1 = np.take_along_axis(grp, idx1[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    vals = np.stack([v0, v1], axis=2).reshape(m, k // 2)
    code = (idx0.astype(np.uint8) | (idx1.astype(np.uint8) << 2)).astype(np.uint8)
    ng = k // 4
    nb = (ng + 1) // 2
    padded = np.zeros((m, 2 * nb), dtype=np.uint8)
    padded[:, :ng] = code
    idx = (padded[:, 0::2] | (padded[:, 1::2] << 4)).astype(np.uint8)
    return vals, idx


def decompress(vals, idx, k: int) -> np.ndarray:
    """Inverse of ``compress``: bf16 words at their channels, zero words
    (+0) at the pruned channels."""
    vals = np.asarray(vals, dtype=np.uint16)
    idx = np.asarray(idx, dtype=np.uint8)
    m = vals.shape[0]
    ng = k // 4
    codes = np.empty((m, 2 * idx.shape[1]), dtype=np.uint8)
    codes[:, 0::2] = idx & 0x0F
    codes[:, 1::2] = idx >> 4
    codes = codes[:, :ng]
    i0 = (codes & 3).astype(np.int64)
    i1 = (codes >> 2).astype(np.int64)
    out = np.zeros((m, ng, 4), dtype=np.uint16)
    pair = vals.reshape(m, ng, 2)
    np.put_along_axis(out, i0[:, :, None], pair[:, :, 0:1], axis=2)
    np.put_along_axis(out, i1[:, :, None], pair[:, :, 1:2], axis=2)
    return out.reshape(m, k)


def dense_linear_ref(x_bits, w_bits) -> np.ndarray:
    """Dense baseline Y = X W^T in fp64 (qingkeai article, section 02 and
    section 05's dense-GEMM comparison)."""
    return bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(w_bits).T


def lora_down_ref(x_bits, a_bits) -> np.ndarray:
    """T = (X - S(X)) A^T: the LoRA branch's input is the pruned residual
    (qingkeai article, section 03.2)."""
    x = bf16_bits_to_f64(x_bits)
    sx = sparsify(x_bits)[0]
    return (x - sx) @ bf16_bits_to_f64(a_bits).T


def sparse_linear_ref(x_bits, w_bits, a_bits=None, b_bits=None, alpha: float = 1.0):
    """Y = S(X) W^T + alpha * ((X - S(X)) A^T) B^T in fp64, S(X) as a dense
    masked matrix (qingkeai article, sections 02, 03.2 and 04)."""
    x = bf16_bits_to_f64(x_bits)
    sx = sparsify(x_bits)[0]
    y = sx @ bf16_bits_to_f64(w_bits).T
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        t = (x - sx) @ bf16_bits_to_f64(a_bits).T
        y = y + alpha * (t @ bf16_bits_to_f64(b_bits).T)
    return y


def sparse_linear_gather_ref(x_bits, w_bits, a_bits=None, b_bits=None, alpha: float = 1.0):
    """The same layer computed from the compressed form, one token at a time:
    s_m * W[:, kept columns of m] @ vals_m, which is what a sparse GEMM does
    with the compressed operand.  The LoRA branch is the same as in
    ``sparse_linear_ref``.  Pure loops over tokens: for small inputs."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    m, k = x_bits.shape
    w = bf16_bits_to_f64(w_bits)
    _, mask, s, idx0, idx1 = sparsify(x_bits)
    vals, _ = compress(x_bits, idx0, idx1)
    v = bf16_bits_to_f64(vals)
    base = np.arange(k // 4) * 4
    y = np.empty((m, w.shape[0]))
    for row in range(m):
        cols = np.stack([base + idx0[row], base + idx1[row]], axis=1).reshape(-1)
        y[row] = s[row] * (w[:, cols] @ v[row])
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        y = y + alpha * (lora_down_ref(x_bits, a_bits) @ bf16_bits_to_f64(b_bits).T)
    return y


def compressed_linear_ref(vals, idx, scale, w_bits, k: int) -> np.ndarray:
    """The structured-sparse product on an activation already in the
    canonical compressed form: Y = diag(scale) decompress(vals, idx) W^T in
    fp64 (qingkeai article, section 04: the sparse GEMM consumes the
    compressed activation; section 02: Y = S(X) W^T with the compensation as
    a per-token factor).  ``scale`` None means 1 (values stored already
    scaled)."""
    xd = bf16_bits_to_f64(decompress(vals, idx, k))
    y = xd @ bf16_bits_to_f64(w_bits).T
    if scale is not None:
        y = y * np.asarray(scale, dtype=np.float64)[:, None]
    return y


# ---------------------------------------------------------------------------
# Compensation and LoRA-input variants the pages leave open.  The default of
# every function above is comp="token", lora="residual".

def round_to_bf16(v) -> np.ndarray:
    """fp64 -> nearest bf16 value (8 significant bits), ties to even, exact:
    v = f 2^e with 0.5 <= |f| < 1, f is rounded to a multiple of 2^-8.  For
    the normal bf16 range (|v| >= 2^-126), which all values here are in."""
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)


def group_compensation_scale(x: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Per group of 4: (L1 of the group) / (L1 of its kept pair), 1 where the
    kept pair is zero (then the whole group is).  [M, K/4]."""
    m, k = x.shape
    ax = np.abs(x).reshape(m, k // 4, 4)
    mk = mask.reshape(m, k // 4, 4)
    lk = np.where(mk, ax, 0.0).sum(axis=2)
    tot = ax.sum(axis=2)
    out = np.ones_like(lk)
    nz = lk > 0
    out[nz] = tot[nz] / lk[nz]
    return out


def sparsify_variant(bits, comp: str = "token"):
    """S(X) under a compensation variant (ai-feeds summary, 核心模块 1 leaves
    the granularity open):

    * "token":  s per token (the default, = ``sparsify``);
    * "none":   no compensation, S(X) = M * X;
    * "tensor": one s for the whole X, (sum of all L1) / (sum of kept L1);
    * "group":  s per group of 4, applied to the kept pair and rounded to
                bf16 (a factor that varies along K can only live in the
                compressed operand itself).

    Returns (S [M, K] fp64, mask)."""
    x = bf16_bits_to_f64(bits)
    mask, _, _ = select_2of4(bits)
    kept = np.where(mask, x, 0.0)
    if comp == "token":
        lk, lp = l1_stats(x, mask)
        return kept * compensation_scale(lk, lp)[:, None], mask
    if comp == "none":
        return kept, mask
    if comp == "tensor":
        lk, lp = l1_stats(x, mask)
        lk_t, lp_t = lk.sum(), lp.sum()
        s = (lk_t + lp_t) / lk_t if lk_t > 0 else 1.0
        return kept * s, mask
    if comp == "group":
        # each kept value times (L1 of its group) / (L1 of its kept pair),
        # rounded once to bf16: formed as (x * L1 group) / L1 kept, an exact
        # product and one division, so that the rounding is that of the
        # exact value; a zero kept pair (a zero group) keeps its zeros
        m, k = x.shape
        ax = np.abs(x).reshape(m, k // 4, 4)
        lk = np.where(mask.reshape(m, k // 4, 4), ax, 0.0).sum(axis=2)
        tot = ax.sum(axis=2)
        lk4 = np.repeat(lk, 4, axis=1)
        tot4 = np.repeat(tot, 4, axis=1)
        nz = lk4 > 0
        q = np.where(nz, kept * tot4 / np.where(nz, lk4, 1.0), kept)
        return round_to_bf16(q), mask
    raise ValueError(comp)


def sparse_linear_variant_ref(x_bits, w_bits, a_bits=None, b_bits=None, alpha: float = 1.0,
                              comp: str = "token", lora: str = "residual"):
    """Y = S(X) W^T + alpha (R A^T) B^T in fp64 with S from
    ``sparsify_variant(comp)`` and the LoRA input R (qingkeai article, 03.2,
    says the branch restores the pruned information; which tensor carries it
    is open):

    * "residual": R = X - S(X) (the default);
    * "pruned":   R = (1 - M) * X, the pruned values only;
    * "input":    R = X, a plain LoRA beside the sparse product."""
    x = bf16_bits_to_f64(x_bits)
    sx, mask = sparsify_variant(x_bits, comp)
    y = sx @ bf16_bits_to_f64(w_bits).T
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        if lora == "residual":
            rin = x - sx
        elif lora == "pruned":
            rin = np.where(mask, 0.0, x)
        elif lora == "input":
            rin = x
        else:
            raise ValueError(lora)
        y = y + alpha * ((rin @ bf16_bits_to_f64(a_bits).T) @ bf16_bits_to_f64(b_bits).T)
    return y
