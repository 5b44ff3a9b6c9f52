"""GPU parity of the fused path's own selection: what the pre-pass of
rtl_sparse_linear writes into its workspace, decoded on the host and
compared with the oracle.

The pre-pass makes the 2:4 pattern decision, Top-K selection, compression and
operand layout generation of the fused kernel (qingkeai RT-Lynx article,
section 04), the per-token compensation scale (ai-feeds summary, 方法 /
核心模块 1) and the LoRA-down product of the pruned residual (qingkeai
article, section 03.2).  Its output never passes through the canonical
compressed format of rtl_sparsify_2of4, so it is checked here directly:

* kept values (unscaled) and 2-bit positions: bit-exact against
  oracle.compress / oracle.select_2of4 (per-group compensation: the folded
  values bit-exact against oracle.sparsify_variant's);
* per-token scale: |s - s_ref| <= 1e-5 s_ref; padding tokens s = 1;
* alpha T / s (stored as a bf16 hi + lo pair): within the worst-case fp32
  summation bound K u (|X| |A|^T + s |M*X| |A|^T) alpha / s (u = 2^-24; the
  kernels form T = X A^T - s (M*X) A^T or ((1-M)*X) A^T + (1-s) (M*X) A^T in
  fp32, K products per sum) plus the hi + lo representation (2^-16 relative);
  rank columns past r exactly zero.

Workspace layout (the pre-pass's operand order for the matrix cores; rows
padded to mp = 256 ceil(M / 256), channels to kp = 128 ceil(K / 128), rank to
rp = 32 ceil(r / 32), each region 256-byte aligned, in this order):

* xv, mp kp bytes: [mp / 128][kp / 64][8][64 lanes][8 bf16] -- group of 8
  16-token blocks, 64-channel k-step, block in the group, lane l = token
  l % 16 of the block with the kept pairs of channels 16 (l / 16) + [0, 16);
* xi, mp kp / 8 bytes: [mp / 128][kp / 64][64 lanes][8 blocks] x uint16 --
  the lane's four group codes idx0 | idx1 << 2, group j in bits 4j..4j+3;
* s, 4 mp bytes: fp32 per token;
* t, 4 mp rp bytes: [mp / 16][rp / 32][hi, lo][64 lanes][8 bf16] -- lane l
  = token l % 16, rank columns 32 rs + 8 (l / 16) + [0, 8).
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
U = 2.0 ** -24


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def rup(v, m):
    return (v + m - 1) // m * m


def layout(m, k, r):
    mp, kp, rp = rup(m, 256), rup(k, 128), rup(r, 32)
    off_xv = 0
    off_xi = rup(off_xv + mp * kp, 256)
    off_s = rup(off_xi + mp * kp // 8, 256)
    off_t = rup(off_s + 4 * mp, 256)
    total = rup(off_t + 4 * mp * rp, 256)
    return mp, kp, rp, off_xv, off_xi, off_s, off_t, total


def decode_workspace(ws: np.ndarray, m, k, r):
    """(vals [mp, kp/2] uint16, codes [mp, kp/4] uint8, s [mp] fp32,
    t [mp, rp] fp64 = hi + lo) from the raw workspace bytes."""
    mp, kp, rp, oxv, oxi, os_, ot, total = layout(m, k, r)
    assert ws.size >= total
    g, ks = mp // 128, kp // 64
    xv = ws[oxv:oxv + mp * kp].view(np.uint16).reshape(g, ks, 8, 4, 16, 8)
    vals = xv.transpose(0, 2, 4, 1, 3, 5).reshape(mp, kp // 2)
    xi = ws[oxi:oxi + mp * kp // 8].view(np.uint16).reshape(g, ks, 4, 16, 8)
    words = xi.transpose(0, 4, 3, 1, 2).reshape(mp, ks * 4)          # 4 groups per word
    codes = np.stack([(words >> (4 * j)) & 0xF for j in range(4)], axis=2).reshape(mp, kp // 4)
    s = ws[os_:os_ + 4 * mp].view(np.float32).copy()
    t = None
    if r > 0:
        tb = ws[ot:ot + 4 * mp * rp].view(np.uint16).reshape(mp // 16, rp // 32, 2, 4, 16, 8)
        tf = oracle.bf16_bits_to_f64(tb)
        tv = tf[:, :, 0] + tf[:, :, 1]                                  # [mb, rs, q, tok, j]
        t = tv.transpose(0, 3, 1, 2, 4).reshape(mp, rp)
    return vals, codes.astype(np.uint8), s, t


def run_prepare(x, a, alpha, variant=0):
    m, k = x.shape
    r = 0 if a is None else a.shape[0]
    need = rtl.sparse_linear_workspace_bytes(m, k, r)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)   # no zeros left by chance
    rtl.prepare(to_dev(x), None if a is None else to_dev(a), alpha, workspace=ws, variant=variant)
    torch.cuda.synchronize()
    return ws.cpu().numpy()


def check_workspace(x, a, alpha=1.0, comp="token", what=""):
    """Decodes the pre-pass workspace for x [M, K] (bf16 bits), LoRA-down a
    [r, K] or None, and checks it against the oracle."""
    m, k = x.shape
    r = 0 if a is None else a.shape[0]
    variant = {"token": rtl.COMP_TOKEN, "group": rtl.COMP_GROUP}[comp]
    ws = run_prepare(x, a, alpha, variant)
    vals, codes, s, t = decode_workspace(ws, m, k, r)
    mp, kp, rp = layout(m, k, r)[:3]
    mask, i0, i1 = oracle.select_2of4(x)
    v_ref, _ = oracle.compress(x, i0, i1)
    code_ref = (i0 | (i1 << 2)).astype(np.uint8)
    ng = k // 4
    bad = codes[:m, :ng] != code_ref
    if bad.any():
        row, grp = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} group codes differ; first at token {row} group {grp}: "
                             f"got {codes[row, grp]} want {code_ref[row, grp]} "
                             f"(x = {x[row, 4 * grp:4 * grp + 4]})")
    got_v = vals[:m, :k // 2]
    if comp == "token":
        badv = got_v != v_ref
        assert not badv.any(), f"{what}: {badv.sum()} kept values differ (first at {np.argwhere(badv)[0]})"
        _, _, s_ref, _, _ = oracle.sparsify(x)
        np.testing.assert_allclose(s[:m].astype(np.float64), s_ref, rtol=1e-5, atol=0, err_msg=what)
    else:
        # the kept values times their group's factor, rounded once to bf16:
        # the same bf16 values as the oracle's
        sx_g, _ = oracle.sparsify_variant(x, "group")
        want = sx_g.reshape(m, k // 4, 4)
        kept_vals = np.stack([np.take_along_axis(want, i0[:, :, None].astype(np.int64), axis=2)[:, :, 0],
                              np.take_along_axis(want, i1[:, :, None].astype(np.int64), axis=2)[:, :, 0]],
                             axis=2).reshape(m, k // 2)
        got = oracle.bf16_bits_to_f64(got_v)
        badf = got != kept_vals
        assert not badf.any(), (f"{what}: {badf.sum()} folded values differ from the oracle's "
                                f"(first at {np.argwhere(badf)[0]})")
        assert (s[:m] == 1.0).all(), f"{what}: per-group compensation leaves s = 1"
        s_ref = np.ones(m)
    assert (s[m:] == 1.0).all(), f"{what}: padding tokens must have s = 1"
    if r == 0:
        return
    xf = oracle.bf16_bits_to_f64(x)
    af = oracle.bf16_bits_to_f64(a)
    sx, _ = oracle.sparsify_variant(x, comp)
    t_ref = (xf - sx) @ af.T
    want = alpha * t_ref / s_ref[:, None]
    kept_abs = np.where(mask, np.abs(xf), 0.0)
    bound = np.abs(xf) @ np.abs(af).T + s_ref[:, None] * (kept_abs @ np.abs(af).T)
    if comp == "group":
        bound = bound + np.abs(sx) @ np.abs(af).T
    tol = abs(alpha) / s_ref[:, None] * (k * U * bound) + 2.0 ** -16 * np.abs(want) + 1e-30
    err = np.abs(t[:m, :r] - want)
    if (err > tol).any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: alpha T / s out of bound at {i}: got {t[:m, :r][i]!r} want {want[i]!r} "
                             f"tol {tol[i]!r}")
    assert (t[:, r:] == 0).all(), f"{what}: rank columns past r must be zero"


# Every instance of the DMA-streamed pre-pass (K % 8 == 0, 0 < r <= 64):
# ranks 32 and 64 (2 or 4 column blocks), K % 128 == 0 (scalar-stepped
# copies) or only K % 8 == 0 (per-step guarded copies), per-token or
# per-group compensation; plus the generic pre-pass (r = 0, r > 64,
# K % 8 == 4).
DMA_CASES = [
    # (M, K, r, comp)
    (300, 1024, 64, "token"), (300, 1024, 64, "group"),
    (300, 1032, 64, "token"), (300, 1032, 64, "group"),
    (130, 2048, 32, "token"), (130, 2048, 32, "group"),
    (130, 1160, 24, "token"), (130, 1160, 24, "group"),
    (48, 128, 64, "token"), (20, 192, 40, "token"),
    (257, 3072, 64, "token"), (1, 3072, 64, "token"),
]
GENERIC_CASES = [
    (300, 1024, 0, "token"), (300, 1028, 64, "token"), (160, 2048, 128, "token"), (64, 260, 96, "group"),
]


@pytest.mark.parametrize("case", DMA_CASES + GENERIC_CASES, ids=lambda c: "x".join(map(str, c)))
def test_prepass_workspace_mixture(case):
    m, k, r, comp = case
    say(f"[parity] workspace M={m} K={k} r={r} comp={comp}")
    rng = np.random.default_rng(m * 5 + k + r)
    x = gen.mixture_bernoulli(rng, m, k)
    a = gen.gaussian_bits(rng, (r, k), 0.05) if r else None
    check_workspace(x, a, 0.75, comp, f"mixture {case}")


@pytest.mark.parametrize("case", DMA_CASES + GENERIC_CASES, ids=lambda c: "x".join(map(str, c)))
def test_prepass_workspace_tie_heavy(case):
    """Values from {0, -0, +-1, +-2, +-4}: most groups tie at the keep/prune
    boundary, which both sides resolve toward the lower channel."""
    m, k, r, comp = case
    say(f"[parity] workspace tie-heavy M={m} K={k} r={r} comp={comp}")
    rng = np.random.default_rng(m * 11 + k + 3 * r)
    x = gen.tie_heavy(rng, m, k)
    a = gen.gaussian_bits(rng, (r, k), 0.05) if r else None
    check_workspace(x, a, 1.0, comp, f"tie-heavy {case}")


@pytest.mark.parametrize("k,r", [(1024, 64), (1032, 32), (1028, 64)], ids=lambda v: str(v))
def test_prepass_workspace_subnormal_and_zero_rows(k, r):
    """Rows of bf16 subnormals, a row mixing them with normal values, all-zero
    and all -0 rows, rows with at most two non-zeros per group."""
    rng = np.random.default_rng(k + r)
    m = 96
    x = gen.mixture_bernoulli(rng, m, k)
    sub = (rng.integers(1, 128, size=(4, k)) | (rng.integers(0, 2, size=(4, k)) << 15)).astype(np.uint16)
    x[0:4] = sub
    x[4] = np.where(rng.random(k) < 0.5, sub[0], x[4])
    x[5] = 0
    x[6] = 0x8000
    x[16:32] = gen.at_most_two_nonzero(rng, 16, k)
    a = gen.gaussian_bits(rng, (r, k), 0.05)
    check_workspace(x, a, 1.0, "token", f"subnormal K={k} r={r}")
    _, _, scale, _, _ = oracle.sparsify(x[16:32])
    assert (scale == 1.0).all()


FULL = ["attn_proj", "mlp_up", "mlp_down", "textimg_p05", "textimg_p10", "textimg_p25",
        "mlp_up_share8", "textimg_share8", "textimg_share2"]


@pytest.mark.parametrize("name", FULL)
def test_prepass_workspace_full_size(name):
    """The headline pre-pass at every full workload size, in the launch
    configuration the layer uses."""
    cfg = gen.config(name)
    say(f"[parity] workspace full {name}: M={cfg.m} K={cfg.k} r={cfg.r}")
    x, _, a, _ = gen.make_config(name)
    check_workspace(x, a, 1.0, "token", f"full {name}")


def test_identity_weight_rank64_exposes_fused_mask():
    """W = I with a rank-64 LoRA whose up factor B is zero: the layer runs
    the DMA pre-pass and the LoRA ring steps, and Y = bf16(s * (M*X)), so the
    fused path's own mask shows as Y != 0 wherever x != 0 -- on tie-heavy X."""
    rng = np.random.default_rng(64)
    for k in (256, 1024, 1032):
        say(f"[parity] W = I, r = 64, K={k}")
        x = gen.tie_heavy(rng, 200, k)
        w = gen.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
        a = gen.gaussian_bits(rng, (64, k), 0.05)
        b = np.zeros((k, 64), dtype=np.uint16)
        y = rtl.sparse_linear(to_dev(x), to_dev(w), to_dev(a), to_dev(b))
        torch.cuda.synchronize()
        yh = oracle.bf16_bits_to_f64(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        sx, mask, s, _, _ = oracle.sparsify(x)
        nz = oracle.bf16_bits_to_f64(x) != 0
        assert np.array_equal((yh != 0)[nz], mask[nz]), f"K={k}: fused mask differs"
        assert ((yh != 0) <= mask).all(), f"K={k}: a pruned channel reached Y"
        # s * x rounded once to bf16 (s in fp32 on the GPU: within one ulp)
        ulp = np.ldexp(1.0, np.frexp(np.abs(sx))[1] - 8)
        assert (np.abs(yh - sx) <= ulp).all(), f"K={k}: Y != bf16(s x)"
