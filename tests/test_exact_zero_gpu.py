"""GPU parity where fp32 accumulation is stressed: weights that are exactly
zero, and activations with a large common offset, an outlier channel or a
huge magnitude, through every launch configuration of the library.

The oracle's rule for an output that is exactly zero is exact equality
("We're Teaching Your Browser to Paint", section "The lucky break that
wasn't luck": code 1 is weight (1 - 1) * d = 0, so a weight of all 1 codes is
W = 0 and y = x W^T = 0).  The kernels start each block's sum at -1.25 S and
add x (1 + c / 4); those two sums round differently, so they must recognise
an all-zero block and add nothing for it.  Likewise a 4-bit group whose codes
all equal an integer zero point ((q - z) * s = 0, "We're Teaching...",
section "What's left").  Everything else is held to the usual tolerance of
the oracle.
"""
import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
import ternary_weight_quantized_q2_amd as q2
from ternary_weight_quantized_q2_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU; they must not be skipped silently"
    torch.cuda.set_device(0)
    q2.load()
    yield


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_bits(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV).view(dtype)


def assert_close(y, ref, what=""):
    r = O.acceptance(np.asarray(y, np.float64), ref)
    assert r["ok"], f"{what}: rel_l2={r['rel_l2']:.3e} row_ratio={r['row_ratio']:.3e}"


GEMM_CFGS = ["w48x192", "w96x192", "w64x128", "w32x128", "w32x64",
             "kg2x1x4", "kg4x2x2", "kg2x1x2", "kg2x2x4", "kg2x2x2", "kg2x1x4r3", "kg6x3x2"]
# (path, tile, K split): the GEMV, every GEMM configuration whole, every K-group configuration split
LAUNCHES = ([("gemv", None, 0)] + [("gemm", c, 1) for c in GEMM_CFGS] +
            [("gemm", c, 2) for c in GEMM_CFGS if c.startswith("kg")])
LAUNCH_IDS = [p if t is None else f"{t}-k{s}" for p, t, s in LAUNCHES]
N, K = 333, 1408          # ragged N; 11 blocks, so the last K set of every configuration is partial


def rows_for(path, tile):
    if path == "gemv":
        return 13
    return 75


def zero_weight(n, k, seed, zero_rows=None):
    """Q2_0 codes and f32 scales where the rows in zero_rows (all rows when
    None) have every code 1, so their weights are exactly 0 whatever the
    (non-zero) scales; the other rows are the usual random codes."""
    codes = I.q2_codes(seed, n, k)
    if zero_rows is None:
        codes[:] = 1
    else:
        codes[zero_rows] = 1
    scales = I.q2_scales(seed, n, k) + np.float32(0.25)      # never zero, so only the codes make W = 0
    return codes, scales.astype(np.float16).astype(np.float32)


def packed(codes, scales):
    p, s = q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    p_ref, s_ref = O.pack_q2(codes, scales)
    return p, s, p_ref, s_ref


def x_regime(seed, m, k, regime):
    xb = I.activations_regime_bf16(seed, m, k, regime)
    return xb, dev_bits(xb, torch.bfloat16)


@pytest.mark.parametrize("path,tile,ksplit", LAUNCHES, ids=LAUNCH_IDS)
def test_zero_weight_is_exactly_zero(path, tile, ksplit, force):
    force(path=path, tile=tile, ksplit=ksplit)
    m = rows_for(path, tile)
    codes, scales = zero_weight(N, K, 101)
    p, s, p_ref, s_ref = packed(codes, scales)
    assert not np.any(O.unpack_q2(p_ref, s_ref))                        # the oracle's W is 0
    xb, x = x_regime(102, m, K, "mean8")                               # |S| ~ 1000 per block
    y = torch.full((m, N), float("nan"), device=DEV)
    q2.q2_linear(x, p, s, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0), f"W = 0 must give y = 0 exactly; max |y| = {y.abs().max().item():.3e}"


@pytest.mark.parametrize("path,tile,ksplit", LAUNCHES, ids=LAUNCH_IDS)
def test_zero_weight_rows_among_others(path, tile, ksplit, force):
    """Every third weight row all zero: those output columns exactly 0, the
    rest within tolerance."""
    force(path=path, tile=tile, ksplit=ksplit)
    m = rows_for(path, tile)
    zr = np.arange(0, N, 3)
    codes, scales = zero_weight(N, K, 103, zero_rows=zr)
    p, s, p_ref, s_ref = packed(codes, scales)
    xb, x = x_regime(104, m, K, "mean8")
    y = q2.q2_linear(x, p, s).cpu().numpy()
    ref = O.q2_linear(xb, p_ref, s_ref)
    assert not np.any(ref[:, zr])
    assert not np.any(y[:, zr]), "all-zero weight rows must give exact zeros"
    assert_close(y, ref, f"zero rows among others, {path} {tile} k{ksplit}")


@pytest.mark.parametrize("regime", I.ACT_REGIMES)
@pytest.mark.parametrize("path,tile,ksplit", LAUNCHES, ids=LAUNCH_IDS)
def test_activation_regimes(path, tile, ksplit, regime, force):
    """x = N(8, 1), one channel at 2^12, rows scaled by 2^100 or 2^116, on the
    usual random Q2_0 and 4-bit weights."""
    force(path=path, tile=tile, ksplit=ksplit)
    m = rows_for(path, tile)
    codes, scales = I.q2_codes(105, N, K), I.q2_scales(105, N, K)
    p, s, p_ref, s_ref = packed(codes, scales)
    xb, x = x_regime(106, m, K, regime)
    y = q2.q2_linear(x, p, s).cpu().numpy()
    assert np.all(np.isfinite(y))
    assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"Q2_0 {regime}, {path} {tile} k{ksplit}")
    p4, s4, z4 = I.q4_weights(107, N, K)
    y4 = q2.q4_linear(x, dev_u8(p4), dev_bits(s4, torch.float16), dev_bits(z4, torch.float16)).cpu().numpy()
    assert np.all(np.isfinite(y4))
    assert_close(y4, O.q4_linear(xb, p4, s4, z4), f"4-bit {regime}, {path} {tile} k{ksplit}")


def q4_zero_groups(n, k, seed):
    """4-bit weights where every group of the even rows has all codes equal to
    an integer zero point (weights exactly 0), and the odd rows are random
    codes with random integer zero points (no zero block in general)."""
    rng = np.random.default_rng(seed)
    zi = rng.integers(0, 16, size=(n, k // 128))
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    codes[0::2] = np.repeat(zi[0::2], 128, axis=1)
    p4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = I.f32_to_f16_bits((np.abs(rng.standard_normal((n, k // 128))) * 0.02 + 0.01).astype(np.float32))
    z = I.f32_to_f16_bits(zi.astype(np.float32))
    return p4, s, z


@pytest.mark.parametrize("path,tile,ksplit", LAUNCHES, ids=LAUNCH_IDS)
def test_q4_zero_groups_are_exactly_zero(path, tile, ksplit, force):
    force(path=path, tile=tile, ksplit=ksplit)
    m = rows_for(path, tile)
    p4, s, z = q4_zero_groups(N, K, 108)
    ref_w = O.unpack_q4(p4, s, z)
    assert not np.any(ref_w[0::2]) and np.all(np.any(ref_w[1::2], axis=1))
    xb, x = x_regime(109, m, K, "mean8")
    y = q2.q4_linear(x, dev_u8(p4), dev_bits(s, torch.float16), dev_bits(z, torch.float16)).cpu().numpy()
    assert not np.any(y[:, 0::2]), "4-bit groups of codes equal to the zero point must add exactly nothing"
    assert_close(y, O.q4_linear(xb, p4, s, z), f"4-bit zero groups, {path} {tile} k{ksplit}")


def test_q4_non_integer_zero_point_is_not_zero(force):
    """Codes all 7 with zero point 7.5 (not an integer): no weight is zero, and
    the group must not be taken for a zero one."""
    force(path="gemm", tile="kg2x1x4")
    n, k, m = 64, 256, 40
    p4 = np.full((n, k // 2), 0x77, np.uint8)
    s = np.full((n, k // 128), 0x3C00, np.uint16)                       # 1.0
    z = np.full((n, k // 128), I.f32_to_f16_bits(np.float32([7.5]))[0], np.uint16)
    xb, x = x_regime(110, m, k, "mean8")
    y = q2.q4_linear(x, dev_u8(p4), dev_bits(s, torch.float16), dev_bits(z, torch.float16)).cpu().numpy()
    assert_close(y, O.q4_linear(xb, p4, s, z), "4-bit non-integer zero point")
    assert np.all(y != 0)


LR_LAUNCHES = [("gemv", None), ("gemm", "kg6x3x2"), ("gemm", "w48x192"), ("gemm", "w96x192"), ("gemm", "w64x128"),
               ("gemm", "w32x128"), ("gemm", "w32x64"), ("auto", None)]


@pytest.mark.parametrize("path,tile", LR_LAUNCHES, ids=[p if t is None else t for p, t in LR_LAUNCHES])
def test_lowrank_on_zero_weight_is_the_branch(path, tile, force):
    """W = 0 (all codes 1): y is the branch (x A^T) B^T alone, within tolerance of
    the oracle's two float64 products; and r = 0 gives exact zeros."""
    force(path=path, tile=tile)
    m = 13 if path == "gemv" else (192 if path == "auto" else rows_for(path, tile))
    r = 32
    codes, scales = zero_weight(N, K, 111)
    p, s, p_ref, s_ref = packed(codes, scales)
    xb, x = x_regime(112, m, K, "mean8")
    a, b = I.lowrank_factors(113, r, K, N)
    y = q2.q2_linear_lowrank(x, p, s, dev_bits(a, torch.float16), dev_bits(b, torch.float16)).cpu().numpy()
    ref = O.q2_linear_lowrank(xb, p_ref, s_ref, a, b)
    assert_close(y, ref, f"branch on W = 0, {path} {tile}")
    y0 = q2.q2_linear_ex(x, p, s).cpu().numpy()
    assert not np.any(y0)


@pytest.mark.parametrize("path,tile", [("gemv", None), ("gemm", "kg6x3x2"), ("gemm", "w32x64")])
def test_accumulate_zero_weight_keeps_y(path, tile, force):
    force(path=path, tile=tile)
    m = rows_for(path, tile)
    codes, scales = zero_weight(N, K, 114)
    p, s, _, _ = packed(codes, scales)
    _, x = x_regime(115, m, K, "mean8")
    y0 = torch.randn((m, N), device=DEV)
    y = y0.clone()
    q2.q2_linear_ex(x, p, s, y=y, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y0), "adding a zero product must leave y unchanged"


A8_ZERO = [("a8_6x3x2", 1), ("a8_6x3x2", 2), ("a8_1x2x4", 1), ("a8_2x1x4", 2), ("a8_6x3x1r3", 1)]


@pytest.mark.parametrize("tile,ksplit", A8_ZERO)
def test_a8_zero_weight_is_exactly_zero(tile, ksplit, force):
    """8-bit activations: a block sum of codes times (1 - 1) is the integer 0,
    so W = 0 gives y = 0, and all-zero rows among others give zero columns."""
    force(tile=tile, ksplit=ksplit)
    m = 75
    codes, scales = zero_weight(N, K, 116)
    p, s, _, _ = packed(codes, scales)
    _, x = x_regime(117, m, K, "mean8")
    y = q2.q2_linear_a8(x, p, s)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    zr = np.arange(1, N, 4)
    codes, scales = zero_weight(N, K, 118, zero_rows=zr)
    p, s, p_ref, s_ref = packed(codes, scales)
    xb, x = x_regime(119, m, K, "outlier")
    y = q2.q2_linear_a8(x, p, s).cpu().numpy()
    assert not np.any(y[:, zr])
    assert_close(y, O.q2_linear_a8(xb, p_ref, s_ref), f"a8 zero rows among others, {tile} k{ksplit}")
