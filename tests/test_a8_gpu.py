"""GPU parity of the 8-bit activation linear (q2_linear_a8) against the CPU
oracle.  The codes and row scales, which float32 arithmetic decides, must be
bit-exact (both sides divide in IEEE float32 and round half to even); the
product is held to the linear's tolerance against the oracle's y = s * (c W^T).

The workspace holds the codes as int8 [M, K] with every group of 16 codes of
a row stored as a transposed 4 x 4 byte matrix (byte 4 j + i of a group is
code 4 i + j), then the f32 row scales at M * K rounded up to 256 bytes.
"""
import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
import ternary_weight_quantized_q2_amd as q2
from ternary_weight_quantized_q2_amd import inputs as I
from tests.test_parity_gpu import DEV, assert_close, dev_bits, q2_weights, sample_cols

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU; they must not be skipped silently"
    torch.cuda.set_device(0)
    q2.load()
    yield


def a8_inputs(cfg, m, k):
    """bf16 activations with rows of different ranges, a row of zeros and a row with one large value."""
    x = (I.activations_bf16(cfg, m, k).astype(np.uint32) << 16).view(np.float32).copy()
    x[::3] *= 37.0
    if m > 1:
        x[1] = 0.0
    if m > 2:
        x[2, k // 2] = 900.0
    return I.f32_to_bf16_bits(x)


def run_a8(xb, p, s, n):
    m, k = xb.shape
    ws = torch.zeros(max(q2.a8_workspace_bytes(m, k), 1), dtype=torch.uint8, device=DEV)
    y = q2.q2_linear_a8(dev_bits(xb, torch.bfloat16), p, s, workspace=ws)
    torch.cuda.synchronize()
    off = (m * k + 255) // 256 * 256
    stored = ws[:m * k].cpu().numpy().view(np.int8).reshape(m, k // 16, 4, 4)
    codes = stored.transpose(0, 1, 3, 2).reshape(m, k).astype(np.int32)
    scales = ws[off:off + 4 * m].view(torch.float32).cpu().numpy()
    return y.cpu().numpy(), codes, scales


@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (5, 300, 640), (16, 257, 1280), (17, 100, 256), (75, 200, 1408),
                                   (200, 333, 384)])
def test_a8_codes_and_product(m, n, k):
    p, s, p_ref, s_ref = q2_weights(61, n, k)
    xb = a8_inputs(61, m, k)
    y, codes, scales = run_a8(xb, p, s, n)
    q_ref, s8_ref = O.quantize_rows_a8(xb)
    assert np.array_equal(codes, q_ref), "codes"
    assert np.array_equal(scales.view(np.uint32), s8_ref.view(np.uint32)), "row scales"
    assert_close(y, O.q2_linear_a8(xb, p_ref, s_ref), f"a8 M={m} N={n} K={k}")


A8_CFGS = ["a8_6x3x2", "a8_4x2x2", "a8_2x2x2", "a8_2x1x4", "a8_1x2x4", "a8_1x1x4", "a8_8x3x2", "a8_6x3x1r3",
           "a8_4x4x2", "a8_6x3x2r3", "a8_4x2x4", "a8_6x2x2", "a8_4x3x2"]
A8_PATHS = [(c, s) for c in A8_CFGS for s in (1, 2)]


@pytest.mark.parametrize("m", [13, 75, 200])
@pytest.mark.parametrize("cfg,split", A8_PATHS, ids=[f"{c}-k{s}" for c, s in A8_PATHS])
def test_a8_every_config(cfg, split, m, force):
    """Every int8 configuration, whole K and split, on ragged M and N and 11
    blocks of K (the last set of every ring partial)."""
    n, k = 333, 1408
    force(tile=cfg, ksplit=split)
    p, s, p_ref, s_ref = q2_weights(62, n, k)
    xb = a8_inputs(62, m, k)
    y, codes, _ = run_a8(xb, p, s, n)
    assert np.array_equal(codes, O.quantize_rows_a8(xb)[0]), "codes"
    assert_close(y, O.q2_linear_a8(xb, p_ref, s_ref), f"a8 {cfg} split={split} M={m}")


@pytest.mark.parametrize("regime", I.ACT_REGIMES)
@pytest.mark.parametrize("cfg", ["a8_6x3x2", "a8_1x2x4"])
def test_a8_activation_regimes(cfg, regime, force):
    """N(8, 1), an outlier channel at 2^12, and rows near 2^100 and 2^116."""
    m, n, k = 40, 333, 1408
    force(tile=cfg)
    p, s, p_ref, s_ref = q2_weights(66, n, k)
    xb = I.activations_regime_bf16(66, m, k, regime)
    y, codes, scales = run_a8(xb, p, s, n)
    q_ref, s8_ref = O.quantize_rows_a8(xb)
    assert np.array_equal(codes, q_ref), "codes"
    assert np.array_equal(scales.view(np.uint32), s8_ref.view(np.uint32)), "row scales"
    assert np.all(np.isfinite(y))
    assert_close(y, O.q2_linear_a8(xb, p_ref, s_ref), f"a8 {regime} {cfg}")


@pytest.mark.parametrize("m,k,n", [(1536, 3072, 9216), (384, 12288, 3072)])
def test_a8_full_size_sampled(m, k, n):
    p, s, p_ref, s_ref = q2_weights(63, n, k)
    xb = a8_inputs(63, m, k)
    y, _, _ = run_a8(xb, p, s, n)
    cols = sample_cols(n, 96, seed=5)
    q, sc = O.quantize_rows_a8(xb)
    ref = sc.astype(np.float64)[:, None] * (q.astype(np.float64) @ O.unpack_q2(p_ref[cols], s_ref[cols]).T)
    assert_close(y[:, cols], ref, f"a8 M={m} K={k} N={n} sampled")


def test_a8_workspace_errors():
    m, n, k = 4, 64, 256
    p, s, _, _ = q2_weights(64, n, k)
    x = dev_bits(a8_inputs(64, m, k), torch.bfloat16)
    small = torch.zeros(q2.a8_workspace_bytes(m, k) - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear_a8(x, p, s, workspace=small)
    assert e.value.status == q2.Q2_ERR_WORKSPACE


def _extreme_rows(k):
    """bf16 rows at the ends of the 8-bit quantiser's range: ordinary values,
    a row scaled by 1e-30, bf16 subnormals only (the row scale is then an
    fp32 subnormal), values near the bf16 maximum, halves that land exactly on
    rounding ties once divided by s = 1, a constant row and a zero row."""
    g = np.random.default_rng(31)
    x = np.zeros((7, k), np.float32)
    x[0] = g.standard_normal(k)
    x[1] = g.standard_normal(k) * np.float32(1e-30)
    sub = g.integers(0, 128, size=k).astype(np.uint32) | (g.integers(0, 2, size=k).astype(np.uint32) << 15)
    x[2] = (sub << 16).view(np.float32)                     # bf16 subnormals: exponent field 0, random signs
    x[3] = g.standard_normal(k) * np.float32(1e37)
    x[4] = g.integers(-254, 255, size=k).astype(np.float32) / 2
    x[4, 0] = 127.0                                          # amax 127, so s = 1 and x / s keeps the halves
    x[5] = 3.0
    return I.f32_to_bf16_bits(x)


@pytest.mark.parametrize("cfg", ["a8_1x2x4", "a8_2x1x4"])
def test_a8_extreme_rows(cfg, force):
    n, k = 200, 640
    force(tile=cfg)
    p, s, p_ref, s_ref = q2_weights(65, n, k)
    xb = _extreme_rows(k)
    y, codes, scales = run_a8(xb, p, s, n)
    q_ref, s8_ref = O.quantize_rows_a8(xb)
    assert s8_ref[2] > 0 and s8_ref[2] < np.finfo(np.float32).tiny      # the subnormal-scale row is exercised
    assert np.array_equal(codes, q_ref), "codes"
    assert np.array_equal(scales.view(np.uint32), s8_ref.view(np.uint32)), "row scales"
    ref = O.q2_linear_a8(xb, p_ref, s_ref)
    rows = [0, 1, 3, 4, 5, 6]
    assert_close(y[rows], ref[rows], f"a8 extreme rows {cfg}")
    assert not y[6].any()
    # Row 2: the row scale s is an fp32 subnormal, so y = s * v lands in the
    # subnormal range, where fp32 spacing is 2^-149 whatever the value.  The
    # stated bound per output: half that spacing for the final product, plus
    # 1e-4 relative error of v's fp32 sum over its terms' magnitudes (exact
    # integer-code products; far looser than K * 2^-24).  A flush to zero
    # would exceed it.
    w = O.unpack_q2(p_ref, s_ref)
    mag = float(s8_ref[2]) * (np.abs(q_ref[2]).astype(np.float64) @ np.abs(w).T)
    err = np.abs(y[2].astype(np.float64) - ref[2])
    assert np.all(err <= 2.0 ** -150 + 1e-4 * mag), f"row 2: max err {err.max():.3e}"
    assert np.any(y[2] != 0) and np.all(np.abs(ref[2]) < np.finfo(np.float32).tiny * 64)
