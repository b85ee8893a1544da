"""GPU parity at the largest input length the library accepts, K = 2^24, where
the kernels' 32-bit copy and block offsets are closest to their limit.

The GEMV (M = 1), the GEMM (M = 20: a narrow K-group tile split over K) and the
4-bit linear on both paths are checked on sampled output columns against the
oracle, to the linear's tolerance; the device-packed bytes and scale bits of
those rows must equal the oracle's packing.
"""
import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
import ternary_weight_quantized_q2_amd as q2
from ternary_weight_quantized_q2_amd import inputs as I
from tests.test_parity_gpu import DEV, assert_close, dev_bits, dev_u8, host_bits

pytestmark = pytest.mark.gpu

KMAX = 1 << 24
N = 20
COLS = np.array([0, 7, 19])


@pytest.fixture(scope="module")
def x_rows():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU; they must not be skipped silently"
    torch.cuda.set_device(0)
    q2.load()
    return I.activations_bf16(71, 20, KMAX)


@pytest.mark.parametrize("m", [1, 20])
def test_q2_linear_max_k(x_rows, m):
    codes = I.q2_codes_fast(72, N, KMAX)
    scales = I.q2_scales(72, N, KMAX)
    p, s = q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    p_ref, s_ref = O.pack_q2(codes[COLS], scales[COLS])
    del codes
    rows = torch.from_numpy(COLS).to(DEV)
    assert np.array_equal(p[rows].cpu().numpy(), p_ref)
    assert np.array_equal(host_bits(s[rows]), s_ref)
    xb = x_rows[:m]
    y = q2.q2_linear(dev_bits(xb, torch.bfloat16), p, s)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy()[:, COLS], O.q2_linear(xb, p_ref, s_ref), f"Q2_0 M={m} K=2^24")


@pytest.mark.parametrize("m", [1, 20])
def test_q4_linear_max_k(x_rows, m):
    p4, s4, z4 = I.q4_weights(73, N, KMAX)
    xb = x_rows[:m]
    y = q2.q4_linear(dev_bits(xb, torch.bfloat16), dev_u8(p4), dev_bits(s4, torch.float16),
                     dev_bits(z4, torch.float16))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy()[:, COLS], O.q4_linear_cols(xb, p4, s4, z4, COLS), f"4-bit M={m} K=2^24")
