"""The no-allocation variant of the low-rank linear (q2_linear_lowrank_noalloc,
through the C ABI) against the workspace variant (q2_linear_lowrank) on the
same inputs: two calls in a row, the second with smaller sizes, each equal bit
for bit to the workspace variant (the same kernels run) and within tolerance
of the oracle; sizes beyond the fixed scratch are refused."""
import ctypes

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


def bits(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV).view(dtype)


def case(seed, m, n, k, r):
    codes, scales = I.q2_codes(seed, n, k), I.q2_scales(seed, n, k)
    p, s = q2.q2_pack(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    p_ref, s_ref = O.pack_q2(codes, scales)
    xb = I.activations_bf16(seed, m, k)
    a, b = I.lowrank_factors(seed, r, k, n)
    return (bits(xb, torch.bfloat16), p, s, bits(a, torch.float16), bits(b, torch.float16)), \
        O.q2_linear_lowrank(xb, p_ref, s_ref, a, b)


def test_noalloc_matches_workspace_variant_twice():
    # the second call is smaller: it must not see anything of the first call's scratch contents
    for seed, (m, n, k, r) in ((120, (300, 500, 1280, 32)), (121, (40, 200, 640, 8))):
        args, ref = case(seed, m, n, k, r)
        y = torch.full((m, n), float("nan"), device=DEV)
        q2.q2_linear_lowrank_noalloc(*args, y=y)
        y_ws = q2.q2_linear_lowrank(*args)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ws), f"M={m} N={n} K={k} r={r}: differs from q2_linear_lowrank"
        r_acc = O.acceptance(y.cpu().numpy().astype(np.float64), ref)
        assert r_acc["ok"], r_acc


def test_noalloc_gemv_path_and_rank_zero():
    args, ref = case(122, 5, 300, 1024, 16)
    y = q2.q2_linear_lowrank_noalloc(*args)
    assert torch.equal(y, q2.q2_linear_lowrank(*args))
    x, p, s, a, b = args
    a0 = torch.empty((0, 1024), dtype=torch.float16, device=DEV)
    b0 = torch.empty((300, 0), dtype=torch.float16, device=DEV)
    y0 = q2.q2_linear_lowrank_noalloc(x, p, s, a0, b0)
    assert torch.equal(y0, q2.q2_linear(x, p, s))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = q2.load()
    fake = ctypes.c_void_p(1 << 20)
    m, r = 65536, 64                                  # M * r * 4 = 16 MiB > 8 MiB
    st = lib.q2_linear_lowrank_noalloc(fake, fake, fake, fake, fake, r, fake, m, 128, 128,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == q2.Q2_ERR_WORKSPACE
    assert b"scratch" in lib.q2_last_error()
