"""GPU parity: the HIP library (called through its C ABI via the binding)
against the CPU oracle on the same seeded inputs.

Bars: packed bytes, scale bits and dequantised weights bit-exact; outputs
within relative L2 <= 1e-4 over the tensor and, per row, max |err| <= 1e-3 of
the oracle row's RMS.  Where the oracle computes only sampled columns of a
full-size output, the row RMS is taken over those columns.
"""
import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
import ternary_weight_quantized_q2_amd as q2
from ternary_weight_quantized_q2_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU; they must not be skipped silently"
    torch.cuda.set_device(0)
    q2.load()
    yield


DEV = "cuda:0"


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_bits(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV).view(dtype)


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def q2_weights(cfg, n, k):
    """GPU-packed and oracle-packed copies of the same seeded Q2_0 weight."""
    codes = I.q2_codes(cfg, n, k)
    scales = I.q2_scales(cfg, n, k)
    p_dev, s_dev = q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    p_ref, s_ref = O.pack_q2(codes, scales)
    return p_dev, s_dev, p_ref, s_ref


def acts(cfg, m, k):
    xb = I.activations_bf16(cfg, m, k)
    return xb, dev_bits(xb, torch.bfloat16)


def assert_close(y, ref, what=""):
    r = O.acceptance(np.asarray(y, np.float64), ref)
    assert r["ok"], f"{what}: rel_l2={r['rel_l2']:.3e} row_ratio={r['row_ratio']:.3e}"
    return r


def sample_cols(n, count=128, seed=0):
    rng = np.random.default_rng(seed)
    cols = np.concatenate([[0, n - 1], rng.choice(n, min(count, n), replace=False)])
    return np.unique(cols)


@pytest.fixture
def path(request, force):
    p = request.param
    if p != "auto":
        force(path=p)
    else:
        force(path=None)
    return p


# ---------------------------------------------------------------------------
# pack / dequant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(64, 256), (1000, 1280), (9216, 3072)])
def test_pack_bitexact(n, k):
    p_dev, s_dev, p_ref, s_ref = q2_weights(11, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(p_dev.cpu().numpy(), p_ref)
    assert np.array_equal(host_bits(s_dev), s_ref)


def test_pack_errors_report_first_index():
    n, k = 6, 384
    codes = np.ones((n, k), np.uint8)
    scales = np.full((n, k // 128), 0.5, np.float32)
    codes[5, 200] = 3
    codes[4, 7] = 9
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    assert e.value.status == q2.Q2_ERR_CODE and e.value.bad_index == 4 * k + 7
    codes[:] = 2
    scales[2, 1] = 1.000244140625          # not an f16 value
    scales[3, 0] = np.nan
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    assert e.value.status == q2.Q2_ERR_SCALE and e.value.bad_index == 2 * 3 + 1
    scales[2, 1] = 0.5
    scales[3, 0] = 65520.0                  # rounds to infinity in f16
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    assert e.value.status == q2.Q2_ERR_SCALE and e.value.bad_index == 9
    scales[3, 0] = 2.0 ** -24               # smallest f16 subnormal is accepted
    q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))


def test_dequant_exact():
    n, k = 300, 640
    codes = I.q2_codes(12, n, k)
    codes[0, :8] = 3                        # outside the format, decoded by the same formula
    scales = I.q2_scales(12, n, k) * np.where(np.arange(n)[:, None] % 2, -1, 1).astype(np.float32)
    c = codes.reshape(n, k // 4, 4).astype(np.uint32)
    packed = (c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6).astype(np.uint8)
    sc16 = I.f32_to_f16_bits(scales)
    w = q2.q2_dequant(dev_u8(packed), dev_bits(sc16, torch.float16)).cpu().numpy()
    ref = O.unpack_q2(packed, sc16)
    assert np.array_equal(w.astype(np.float64), ref)
    assert not np.any(np.signbit(w[w == 0]))   # zero weights are +0


# ---------------------------------------------------------------------------
# Q2_0 linear
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "gemv", "gemm"], indirect=True)
def test_linear_tiny_config(path):
    c = I.CONFIG_TINY
    p_dev, s_dev, p_ref, s_ref = q2_weights(c["id"], c["N"], c["K"])
    xb, x = acts(c["id"], c["M"], c["K"])
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"tiny {path}")


@pytest.mark.parametrize("path,m", [("gemv", 16), ("gemm", 16), ("auto", 256), ("gemm", 1)], indirect=["path"])
def test_linear_identity_is_exact(path, m):
    k, n = 256, 200
    p_dev, s_dev, p_ref, s_ref = q2_weights(13, n, k)
    eye = np.zeros((m, k), np.float32)
    eye[np.arange(m), np.arange(m)] = 1.0
    y = q2.q2_linear(dev_bits(I.f32_to_bf16_bits(eye), torch.bfloat16), p_dev, s_dev).cpu().numpy()
    w = O.unpack_q2(p_ref, s_ref)
    assert np.array_equal(y.astype(np.float64), w[:, :m].T)


SHAPES = [(1, 1, 128), (1, 17, 384), (3, 130, 1280), (4, 64, 256), (7, 1000, 256), (16, 257, 512), (17, 65, 640),
          (33, 200, 128), (100, 333, 384), (257, 190, 1024), (96, 192, 3072), (300, 450, 2048),
          # the GEMV's twelve-row workgroups (N / 16 below the CU count), with a ragged last workgroup
          (1, 2501, 384), (5, 3070, 640), (16, 4000, 256)]


@pytest.mark.parametrize("path", ["auto", "gemm"], indirect=True)
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_linear_ragged(path, m, n, k):
    p_dev, s_dev, p_ref, s_ref = q2_weights(14, n, k)
    xb, x = acts(14, m, k)
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"{path} M={m} N={n} K={k}")


# Shapes across the automatic configuration choice (several workgroup waves,
# an odd and a single block count, ragged N and, where allowed, ragged M);
# every configuration is also forced in test_forced_gemm_configs.
TILE_CASES = [(192, 24700, 384), (96, 49300, 128), (203, 24700, 384), (500, 8500, 256), (250, 8100, 256),
              (40, 16300, 256), (20, 300, 256)]


@pytest.mark.parametrize("m,n,k", TILE_CASES)
def test_linear_tile_configs(m, n, k):
    p_dev, s_dev, p_ref, s_ref = q2_weights(16, n, k)
    xb, x = acts(16, m, k)
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"M={m} N={n} K={k}")
    p4, s4, z4, xb4, x4, P, S, Z = q4_case(19, m, k, n)
    y4 = q2.q4_linear(x4, P, S, Z).cpu().numpy()
    assert_close(y4, O.q4_linear(xb4, p4, s4, z4), f"q4 M={m} N={n} K={k}")


# Every GEMM kernel configuration, forced through the test-only Q2_GEMM_TILE
# override, on shapes with ragged M and N, block counts that leave the last
# K set partial or shorter than one set, a single block and K = 0.
GEMM_CFGS = ["w48x192", "w96x192", "w64x128", "w32x128", "w32x64",
             "kg2x1x4", "kg4x2x2", "kg2x1x2", "kg2x2x4", "kg2x2x2", "kg2x1x4r3", "kg6x3x2"]
CFG_SHAPES = [(75, 200, 1408), (128, 2560, 384), (33, 1000, 128), (40, 100, 0), (256, 700, 2560), (96, 333, 640)]
_cfg_ref = {}


def _cfg_case(m, n, k):
    key = (m, n, k)
    if key not in _cfg_ref:
        p_dev, s_dev, p_ref, s_ref = q2_weights(21, n, k)
        xb, x = acts(21, m, k)
        p4, s4, z4, xb4, x4, P, S, Z = q4_case(22, m, k, n)
        _cfg_ref[key] = ((x, p_dev, s_dev, O.q2_linear(xb, p_ref, s_ref)),
                         (x4, P, S, Z, O.q4_linear(xb4, p4, s4, z4)))
    return _cfg_ref[key]


@pytest.mark.parametrize("cfg", GEMM_CFGS)
@pytest.mark.parametrize("m,n,k", CFG_SHAPES)
def test_forced_gemm_configs(cfg, m, n, k, force):
    (x, p, s, ref), (x4, P, S, Z, ref4) = _cfg_case(m, n, k)
    force(tile=cfg)
    y = torch.full((m, n), float("nan"), device=DEV)
    q2.q2_linear(x, p, s, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref, f"{cfg} M={m} N={n} K={k}")
    y4 = torch.full((m, n), float("nan"), device=DEV)
    q2.q4_linear(x4, P, S, Z, y4)
    torch.cuda.synchronize()
    assert_close(y4.cpu().numpy(), ref4, f"q4 {cfg} M={m} N={n} K={k}")


@pytest.mark.parametrize("cfg", ["kg6x3x2", "w48x192", "w96x192"])
def test_output_not_16_byte_aligned(cfg, force):
    """y 4 bytes past a 16-byte boundary takes the per-element store path."""
    m, n, k = 192, 400, 640
    (x, p, s, ref), _ = _cfg_case(m, n, k)
    force(tile=cfg)
    flat = torch.full((m * n + 4,), float("nan"), device=DEV)
    y = flat[1:1 + m * n].view(m, n)
    assert y.data_ptr() % 16 == 4
    q2.q2_linear(x, p, s, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref, f"{cfg} unaligned y")
    assert torch.isnan(flat[0]) and torch.isnan(flat[1 + m * n:]).all()


def test_forced_gemm_config_errors(force):
    (x, p, s, _), _ = _cfg_case(75, 200, 1408)
    with pytest.raises(q2.Q2Error) as e:
        force(tile="no-such-tile")
    assert e.value.status == q2.Q2_ERR_ARG
    force(tile=None)                # the refused name changed nothing; the call runs
    q2.q2_linear(x, p, s)
    force(tile="kg6x3x2")        # the K-group branch takes ranks up to 64 only
    p65, s65, _, _, _, x65, _, _, A65, B65 = lowrank_case(24, 40, 256, 100, 65)
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear_lowrank(x65, p65, s65, A65, B65)
    assert e.value.status == q2.Q2_ERR_HIP


KG_CFGS = [c for c in GEMM_CFGS if c.startswith("kg")]


@pytest.mark.parametrize("cfg", KG_CFGS)
@pytest.mark.parametrize("m,n,k", CFG_SHAPES + [(384, 3072, 12288)])
def test_forced_k_split(cfg, m, n, k, force):
    # K in two parts added into a zeroed y; a single block (K = 128) leaves the second part empty
    (x, p, s, ref), (x4, P, S, Z, ref4) = _cfg_case(m, n, k) if k <= 4096 else _k_split_big_case(m, n, k)
    force(tile=cfg)
    force(ksplit=2)
    y = torch.full((m, n), float("nan"), device=DEV)
    q2.q2_linear(x, p, s, y)
    y_again = q2.q2_linear(x, p, s)
    torch.cuda.synchronize()
    assert torch.equal(y, y_again), "a split call must be run-to-run deterministic"
    yh = y.cpu().numpy()
    if isinstance(ref, tuple):              # sampled columns of a full-size shape
        cols, ref_cols = ref
        assert_close(yh[:, cols], ref_cols, f"{cfg} split M={m} N={n} K={k} sampled")
    else:
        assert_close(yh, ref, f"{cfg} split M={m} N={n} K={k}")
    if P is not None:
        y4 = torch.full((m, n), float("nan"), device=DEV)
        q2.q4_linear(x4, P, S, Z, y4)
        torch.cuda.synchronize()
        assert_close(y4.cpu().numpy(), ref4, f"q4 {cfg} split M={m} N={n} K={k}")


_big = {}


def _k_split_big_case(m, n, k):
    if (m, n, k) not in _big:
        p_dev, s_dev, p_ref, s_ref = q2_weights(23, n, k)
        xb, x = acts(23, m, k)
        cols = sample_cols(n, 96, seed=3)
        _big[(m, n, k)] = ((x, p_dev, s_dev, (cols, O.q2_linear_cols(xb, p_ref, s_ref, cols))),
                           (None, None, None, None, None))
    return _big[(m, n, k)]


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_k_split_unaligned_y(offset, force):
    # the zero fill before a split call covers y from any 4-byte position and touches nothing around it
    m, n, k = 75, 201, 1408
    (x, p, s, ref), _ = _cfg_case(m, n, k)
    force(tile="kg2x2x2")
    force(ksplit=2)
    flat = torch.full((m * n + 8,), float("nan"), device=DEV)
    y = flat[offset:offset + m * n].view(m, n)
    q2.q2_linear(x, p, s, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref, f"split, y at +{4 * offset} bytes")
    assert torch.isnan(flat[:offset]).all() and torch.isnan(flat[offset + m * n:]).all()


def test_forced_k_split_errors(force):
    (x, p, s, _), _ = _cfg_case(75, 200, 1408)
    with pytest.raises(q2.Q2Error) as e:
        force(ksplit=3)
    assert e.value.status == q2.Q2_ERR_ARG
    force(ksplit=2)
    force(tile="w32x128")       # only K-group tiles split K
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear(x, p, s)
    assert e.value.status == q2.Q2_ERR_HIP
    force(tile="kg2x2x2")       # an accumulating call cannot split
    y = torch.zeros((75, 200), device=DEV)
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear_ex(x, p, s, y=y, accumulate=True)
    assert e.value.status == q2.Q2_ERR_HIP
    force(path="gemv")          # nor does the GEMV
    xs = x[:8].contiguous()
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear(xs, p, s)
    assert e.value.status == q2.Q2_ERR_HIP


def _offset_f16(t):
    """The same values in a buffer whose first element sits 2 bytes past a 4-byte boundary."""
    flat = torch.empty(t.numel() + 1, dtype=torch.float16, device=t.device)
    v = flat[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 4 == 2
    return v


@pytest.mark.parametrize("m,n,k", [(203, 24700, 384), (130, 700, 1280), (5, 77, 384)])
def test_scales_at_odd_halfword(m, n, k):
    p_dev, s_dev, p_ref, s_ref = q2_weights(17, n, k)
    xb, x = acts(17, m, k)
    y = q2.q2_linear(x, p_dev, _offset_f16(s_dev)).cpu().numpy()
    assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"odd scales M={m} N={n} K={k}")
    p4, s4, z4, xb4, x4, P, S, Z = q4_case(18, m, k, n)
    y4 = q2.q4_linear(x4, P, _offset_f16(S), _offset_f16(Z)).cpu().numpy()
    assert_close(y4, O.q4_linear(xb4, p4, s4, z4), f"odd q4 scales M={m} N={n} K={k}")


def _edge_weight(n, k, regime):
    """Hand-made Q2_0 bytes and f16 scale bits: codes including 3 (outside the
    format, decoded by the same formula) and scales of both signs in one of
    three regimes: "mixed" (ordinary scales with zeros, subnormals and the
    largest finite values interspersed), "subnormal" (every scale an f16
    subnormal, so a flush to zero would show) and "large" (every scale within
    a factor 2 of the largest finite f16)."""
    codes = I.q2_codes(21, n, k)
    codes[0, :40] = 3
    codes[n - 1, k - 130:] = 3
    c = codes.reshape(n, k // 4, 4).astype(np.uint32)
    packed = (c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6).astype(np.uint8)
    rng = np.random.default_rng(23)
    if regime == "subnormal":
        sbits = rng.integers(1, 0x400, size=(n, k // 128)).astype(np.uint16)
    elif regime == "large":
        sbits = rng.integers(0x7800, 0x7C00, size=(n, k // 128)).astype(np.uint16)
    else:
        sbits = I.f32_to_f16_bits(I.q2_scales(21, n, k))
        special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF], np.uint16)
        sbits.reshape(-1)[::7] = np.resize(special, sbits.reshape(-1)[::7].shape)
    sbits[1::2] ^= 0x8000                                  # every other row of the opposite sign
    return packed, sbits


@pytest.mark.parametrize("regime", ["mixed", "subnormal", "large"])
@pytest.mark.parametrize("cfg,m", [("gemv", 1), ("gemv", 13), ("auto", 96), ("w96x192", 192), ("kg6x3x2", 100),
                                   ("kg2x1x4r3", 40), ("w48x192", 75), ("kg2x2x4", 33)])
def test_linear_scale_and_code_extremes(cfg, m, regime, force):
    n, k = 333, 1408
    packed, sbits = _edge_weight(n, k, regime)
    if cfg == "gemv":
        force(path="gemv")
    elif cfg != "auto":
        force(path="gemm")
        force(tile=cfg)
    xb, x = acts(22, m, k)
    y = q2.q2_linear(x, dev_u8(packed), dev_bits(sbits, torch.float16)).cpu().numpy()
    assert np.all(np.isfinite(y))
    assert_close(y, O.q2_linear(xb, packed, sbits), f"{regime} scales and code 3, {cfg} M={m}")


def test_linear_empty_and_k_zero():
    n = 40
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    p = torch.empty((n, 0), dtype=torch.uint8, device=DEV)
    s = torch.empty((n, 0), dtype=torch.float16, device=DEV)
    y = torch.full((5, n), float("nan"), device=DEV)
    q2.q2_linear(x, p, s, y)
    assert torch.all(y == 0)
    y17 = torch.full((17, n), float("nan"), device=DEV)
    q2.q2_linear(torch.empty((17, 0), dtype=torch.bfloat16, device=DEV), p, s, y17)
    assert torch.all(y17 == 0)
    p_dev, s_dev, _, _ = q2_weights(15, n, 256)
    y0 = q2.q2_linear(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), p_dev, s_dev)
    assert y0.shape == (0, n)


@pytest.mark.parametrize("k,n", I.GEMV_SHAPES)
def test_gemv_full_shapes(k, n):
    p_dev, s_dev, p_ref, s_ref = q2_weights(20, n, k)
    for m in (1, 4, 16):
        xb, x = acts(20 + m, m, k)
        y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
        assert_close(y, O.q2_linear(xb, p_ref, s_ref), f"gemv M={m} K={k} N={n}")


@pytest.mark.parametrize("k,n", I.GEMM_SHAPES)
def test_gemm_full_shapes(k, n):
    m = I.GEMM_M
    p_dev, s_dev, p_ref, s_ref = q2_weights(30, n, k)
    xb, x = acts(30, m, k)
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    if (k, n) == (3072, 3072):
        assert_close(y, O.q2_linear(xb, p_ref, s_ref), "gemm full")
    cols = sample_cols(n)
    assert_close(y[:, cols], O.q2_linear_cols(xb, p_ref, s_ref, cols), f"gemm K={k} N={n} sampled")


@pytest.mark.parametrize("m", I.QUARTER_M)
@pytest.mark.parametrize("k,n", I.GEMM_SHAPES)
def test_quarter_step_shapes(m, k, n):
    # the rows of the quarter-size first step, in the launch configuration the automatic choice gives them
    p_dev, s_dev, p_ref, s_ref = q2_weights(31, n, k)
    xb, x = acts(31, m, k)
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    cols = sample_cols(n, seed=m)
    assert_close(y[:, cols], O.q2_linear_cols(xb, p_ref, s_ref, cols), f"M={m} K={k} N={n} sampled")


def test_determinism_and_guards():
    for m, n, k in ((1, 3072, 3072), (1536, 3072, 3072), (9, 1000, 1280)):
        p_dev, s_dev, p_ref, s_ref = q2_weights(40, n, k)
        xb, x = acts(40, m, k)
        guard = 16384
        buf = torch.full((2 * guard + m * n,), float("nan"), device=DEV)
        buf[:guard] = 1234.5
        buf[-guard:] = -4321.5
        y = buf[guard:guard + m * n].view(m, n)
        q2.q2_linear(x, p_dev, s_dev, y)
        y2 = q2.q2_linear(x, p_dev, s_dev)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any(), "output not fully written"
        assert torch.all(buf[:guard] == 1234.5) and torch.all(buf[-guard:] == -4321.5), "write outside y"
        assert torch.equal(y, y2), "not bitwise reproducible"


def _guarded(m, n):
    guard = 16384
    buf = torch.full((2 * guard + m * n,), float("nan"), device=DEV)
    buf[:guard] = 1234.5
    buf[-guard:] = -4321.5
    return buf, buf[guard:guard + m * n].view(m, n), guard


@pytest.mark.parametrize("entry", ["lowrank", "q4_split", "a8", "q2_split"])
def test_determinism_and_guards_other_entry_points(entry):
    # every output element written, nothing outside it touched, and a second call bitwise equal
    if entry == "lowrank":
        m, k, n, r = 1536, 3072, 3072, 32
        p, s, _, _, _, x, _, _, A, B = lowrank_case(41, m, k, n, r)
        call = lambda y: q2.q2_linear_lowrank(x, p, s, A, B, y=y)
    elif entry == "q4_split":                       # long K over few tiles: the two-part K split
        m, k, n = 128, 9728, 2560
        _, _, _, _, x, P, S, Z = q4_case(42, m, k, n)
        call = lambda y: q2.q4_linear(x, P, S, Z, y)
    elif entry == "a8":
        m, k, n = 1536, 3072, 3072
        p, s, _, _ = q2_weights(43, n, k)
        _, x = acts(43, m, k)
        call = lambda y: q2.q2_linear_a8(x, p, s, y=y)
    else:
        m, k, n = 384, 12288, 3072
        p, s, _, _ = q2_weights(44, n, k)
        _, x = acts(44, m, k)
        call = lambda y: q2.q2_linear(x, p, s, y)
    buf, y, guard = _guarded(m, n)
    call(y)
    y2 = call(torch.empty((m, n), device=DEV))
    torch.cuda.synchronize()
    assert not torch.isnan(y).any(), "output not fully written"
    assert torch.all(buf[:guard] == 1234.5) and torch.all(buf[-guard:] == -4321.5), "write outside y"
    assert torch.equal(y, y2), "not bitwise reproducible"


# ---------------------------------------------------------------------------
# low-rank branch
# ---------------------------------------------------------------------------

def lowrank_case(cfg, m, k, n, r):
    p_dev, s_dev, p_ref, s_ref = q2_weights(cfg, n, k)
    xb, x = acts(cfg, m, k)
    a, b = I.lowrank_factors(cfg, r, k, n)
    return p_dev, s_dev, p_ref, s_ref, xb, x, a, b, dev_bits(a, torch.float16), dev_bits(b, torch.float16)


@pytest.mark.parametrize("m,k,n,r", [(4, 256, 64, 4), (4, 256, 64, 32), (1, 3072, 9216, 32), (17, 384, 100, 5),
                                     (16, 1280, 333, 64), (200, 640, 250, 7), (96, 3072, 192, 64),
                                     (257, 512, 300, 72), (100, 256, 70, 8), (33, 1280, 190, 16), (1, 128, 5, 1),
                                     # eight-wave 96x192 tiles: odd block count, a single block
                                     (192, 640, 24700, 32), (96, 128, 49300, 8), (203, 640, 24700, 16)])
def test_lowrank_parity(m, k, n, r):
    p_dev, s_dev, p_ref, s_ref, xb, x, a, b, A, B = lowrank_case(50, m, k, n, r)
    y = q2.q2_linear_lowrank(x, p_dev, s_dev, A, B).cpu().numpy()
    assert_close(y, O.q2_linear_lowrank(xb, p_ref, s_ref, a, b), f"lowrank M={m} K={k} N={n} r={r}")


LR_SHAPES = [(75, 1408, 333), (33, 128, 200), (130, 640, 700)]


@pytest.mark.parametrize("ksplit", [1, 2])
@pytest.mark.parametrize("r", [1, 5, 8, 32, 64])
@pytest.mark.parametrize("cfg", KG_CFGS)
def test_lowrank_every_kgroup_config(cfg, r, ksplit, force):
    """The rank-r branch carried in the prologue of every K-group
    configuration: ragged M and N, ranks that are and are not multiples of 8,
    the K blocks whole and in two parts (of a split tile only the first part
    adds the branch), and B both at an aligned start and 2 bytes off it (the
    byte-run copy of B)."""
    force(path="gemm", tile=cfg, ksplit=ksplit)
    for m, k, n in LR_SHAPES:
        p_dev, s_dev, p_ref, s_ref, xb, x, a, b, A, B = lowrank_case(51, m, k, n, r)
        ref = O.q2_linear_lowrank(xb, p_ref, s_ref, a, b)
        y = q2.q2_linear_lowrank(x, p_dev, s_dev, A, B).cpu().numpy()
        assert_close(y, ref, f"{cfg} k{ksplit} r={r} M={m} K={k} N={n}")
        y_off = q2.q2_linear_lowrank(x, p_dev, s_dev, A, _offset_f16(B)).cpu().numpy()
        assert np.array_equal(y_off, y), f"{cfg} k{ksplit} r={r}: B at an offset start changed the result"


@pytest.mark.parametrize("cfg", KG_CFGS)
def test_lowrank_kgroup_k_zero_and_accumulate(cfg, force):
    force(path="gemm", tile=cfg)
    m, n, r = 70, 300, 24
    p_dev, s_dev, p_ref, s_ref, xb, x, a, b, A, B = lowrank_case(52, m, 512, n, r)
    # K = 0: the branch of an empty x A^T is zero, so y = 0
    x0 = torch.empty((m, 0), dtype=torch.bfloat16, device=DEV)
    y0 = q2.q2_linear_lowrank(x0, torch.empty((n, 0), dtype=torch.uint8, device=DEV),
                              torch.empty((n, 0), dtype=torch.float16, device=DEV),
                              torch.empty((r, 0), dtype=torch.float16, device=DEV), B)
    assert torch.all(y0 == 0)
    base = torch.randn((m, n), device=DEV)
    y = base.clone()
    q2.q2_linear_ex(x, p_dev, s_dev, y=y, A=A, B=B, accumulate=True)
    v = q2.q2_linear_lowrank(x, p_dev, s_dev, A, B)
    assert torch.equal(y, base + v), "accumulation must give y_old + v exactly"
    assert_close(v.cpu().numpy(), O.q2_linear_lowrank(xb, p_ref, s_ref, a, b), f"{cfg} accumulate")


@pytest.mark.parametrize("r", I.LOWRANK["ranks"])
def test_lowrank_full_shape_sampled(r):
    c = I.LOWRANK
    m, k, n = c["M"], c["K"], c["N"]
    p_dev, s_dev, p_ref, s_ref, xb, x, a, b, A, B = lowrank_case(60 + r, m, k, n, r)
    y = q2.q2_linear_lowrank(x, p_dev, s_dev, A, B).cpu().numpy()
    cols = sample_cols(n)
    ref = O.q2_linear_cols(xb, p_ref, s_ref, cols) + O.lowrank_t(xb, a) @ O.f16_to_f64(b[cols]).T
    assert_close(y[:, cols], ref, f"lowrank full r={r}")


def test_lowrank_rank_zero_is_linear():
    p_dev, s_dev, _, _, _, x, _, _, _, B = lowrank_case(70, 40, 512, 96, 3)
    A0 = torch.empty((0, 512), dtype=torch.float16, device=DEV)
    B0 = torch.empty((96, 0), dtype=torch.float16, device=DEV)
    assert torch.equal(q2.q2_linear_lowrank(x, p_dev, s_dev, A0, B0), q2.q2_linear(x, p_dev, s_dev))


@pytest.mark.parametrize("r", I.LOWRANK["ranks"])
def test_layer_list(r):
    """The low-rank layer list: LOWRANK["linears"] distinct rank-r linears (own
    W, A, B) on one shared x, run LOWRANK["steps"] times in one stream.  Every
    output must be bitwise equal to its first-step value, and linears 0, 37 and
    99 match the oracle over the whole output."""
    c = I.LOWRANK
    m, k, n, layers, steps = c["M"], c["K"], c["N"], c["linears"], c["steps"]
    xb, x = acts(900, m, k)
    ws = torch.empty(q2.lowrank_workspace_bytes(m, r), dtype=torch.uint8, device=DEV)
    cfg = lambda i: 1000 * r + i
    weights = []
    for i in range(layers):
        p_dev, s_dev = q2.q2_pack(dev_u8(I.q2_codes_fast(cfg(i), n, k)),
                                  torch.from_numpy(I.q2_scales(cfg(i), n, k)).to(DEV))
        a, b = I.lowrank_factors(cfg(i), r, k, n)
        weights.append((p_dev, s_dev, dev_bits(a, torch.float16), dev_bits(b, torch.float16)))
    first = [torch.empty((m, n), device=DEV) for _ in range(layers)]
    y = torch.empty((m, n), device=DEV)
    for step in range(steps):
        for i, (p_dev, s_dev, A, B) in enumerate(weights):
            q2.q2_linear_lowrank(x, p_dev, s_dev, A, B, y=first[i] if step == 0 else y, workspace=ws)
            if step > 0:
                assert torch.equal(y, first[i]), f"linear {i} of step {step} differs from step 0"
    torch.cuda.synchronize()
    for i in (0, 37, 99):
        p_ref, s_ref = O.pack_q2(I.q2_codes_fast(cfg(i), n, k), I.q2_scales(cfg(i), n, k))
        a, b = I.lowrank_factors(cfg(i), r, k, n)
        assert_close(first[i].cpu().numpy(), O.q2_linear_lowrank(xb, p_ref, s_ref, a, b),
                     f"layer list r={r} linear {i}")


# ---------------------------------------------------------------------------
# 4-bit nibble variant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "gemm"], indirect=True)
def test_q4_hand_nibble_order(path):
    k = 128
    p4 = np.zeros((1, k // 2), np.uint8)
    p4[0, :2] = [0x21, 0x43]
    x = np.zeros((1, k), np.float32)
    x[0, :4] = [1, 10, 100, 1000]
    y = q2.q4_linear(dev_bits(I.f32_to_bf16_bits(x), torch.bfloat16), dev_u8(p4),
                     dev_bits(np.full((1, 1), 0x3C00, np.uint16), torch.float16),
                     dev_bits(np.zeros((1, 1), np.uint16), torch.float16)).cpu().numpy()
    assert y[0, 0] == 4321.0


def q4_case(cfg, m, k, n):
    p4, s, z = I.q4_weights(cfg, n, k)
    xb, x = acts(cfg, m, k)
    return p4, s, z, xb, x, dev_u8(p4), dev_bits(s, torch.float16), dev_bits(z, torch.float16)


@pytest.mark.parametrize("path", ["auto", "gemm"], indirect=True)
@pytest.mark.parametrize("m,n,k", [(1, 64, 256), (5, 77, 384), (16, 300, 1280), (17, 100, 256), (128, 257, 640),
                                   (1, 2501, 384), (9, 3070, 256)])
def test_q4_ragged(path, m, n, k):
    p4, s, z, xb, x, P, S, Z = q4_case(90, m, k, n)
    y = q2.q4_linear(x, P, S, Z).cpu().numpy()
    assert_close(y, O.q4_linear(xb, p4, s, z), f"q4 {path} M={m} N={n} K={k}")


@pytest.mark.parametrize("k,n", I.Q4_SHAPES)
def test_q4_full_shapes(k, n):
    m = I.Q4_M
    p4, s, z, xb, x, P, S, Z = q4_case(95, m, k, n)
    y = q2.q4_linear(x, P, S, Z).cpu().numpy()
    if (k, n) == (2560, 2560):
        assert_close(y, O.q4_linear(xb, p4, s, z), "q4 full")
    cols = sample_cols(n)
    assert_close(y[:, cols], O.q4_linear_cols(xb, p4, s, z, cols), f"q4 K={k} N={n} sampled")


@pytest.mark.parametrize("regime", ["mixed", "subnormal", "large"])
@pytest.mark.parametrize("cfg,m", [("gemv", 1), ("gemv", 11), ("auto", 128), ("kg4x2x2", 70), ("kg2x2x4", 33),
                                   ("w48x192", 96)])
def test_q4_scale_and_zero_extremes(cfg, m, regime, force):
    """4-bit weights with scales of both signs in the three regimes of the Q2_0
    case, and zero points that are zero, negative, non-integer, f16
    subnormals or far outside the code range (the accumulator start
    -(1 + z/16) S then dominates the block sum)."""
    n, k = 257, 1408
    p4, _, _ = I.q4_weights(24, n, k)
    _, sbits = _edge_weight(n, k, regime)
    rng = np.random.default_rng(25)
    z = rng.uniform(-16.0, 31.0, size=(n, k // 128)).astype(np.float32)
    zbits = I.f32_to_f16_bits(z)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7BFF, 0xFBFF, 0x3C00, 0x4B80], np.uint16)
    zbits.reshape(-1)[::5] = np.resize(special, zbits.reshape(-1)[::5].shape)
    if cfg == "gemv":
        force(path="gemv")
    elif cfg != "auto":
        force(path="gemm")
        force(tile=cfg)
    xb, x = acts(26, m, k)
    y = q2.q4_linear(x, dev_u8(p4), dev_bits(sbits, torch.float16), dev_bits(zbits, torch.float16)).cpu().numpy()
    assert np.all(np.isfinite(y))
    assert_close(y, O.q4_linear(xb, p4, sbits, zbits), f"4-bit {regime} scales, extreme zeros, {cfg} M={m}")


def _lowrank_regime(shape, regime, seed):
    """f16 bits of one low-rank factor, with random signs: ordinary
    N(0, 0.02) values, all f16 subnormals, or magnitudes in [32768, 65504],
    within a factor 2 of the largest finite f16 (the branch then reaches
    ~1e12, well inside fp32)."""
    rng = np.random.default_rng(seed)
    if regime == "subnormal":
        b = rng.integers(1, 0x400, size=shape).astype(np.uint16)
    elif regime == "large":
        b = rng.integers(0x7800, 0x7C00, size=shape).astype(np.uint16)
    else:
        b = I.f32_to_f16_bits((rng.standard_normal(shape) * 0.02).astype(np.float32))
    return b ^ (rng.integers(0, 2, size=shape).astype(np.uint16) << 15)


@pytest.mark.parametrize("regime", ["ordinary", "subnormal", "large"])
@pytest.mark.parametrize("cfg,m,r", [("gemv", 3, 32), ("gemv", 16, 5), ("auto", 192, 32), ("kg6x3x2", 96, 64),
                                     ("w48x192", 75, 32), ("w64x128", 40, 8), ("w32x64", 33, 5)])
def test_lowrank_branch_alone_extremes(cfg, m, r, regime, force):
    """Every code 1, so W = 0 exactly whatever the (non-zero) block scales and
    y is the branch (x A^T) B^T alone, with the factors in the three
    regimes; the branch's bf16 limb arithmetic is then the whole result.  This
    needs the kernels to add exactly nothing for an all-zero block (their
    offset-started block sums would otherwise leave fp32 noise of the size of
    x d, above the subnormal-regime branch)."""
    n, k = 300, 640
    codes = np.ones((n, k), np.uint8)
    scales = (I.q2_scales(27, n, k) + np.float32(0.5)).astype(np.float16).astype(np.float32)
    p = q2.q2_pack(dev_u8(codes), torch.from_numpy(scales).to(DEV))
    p_ref, s_ref = O.pack_q2(codes, scales)
    a = _lowrank_regime((r, k), regime, 28)
    b = _lowrank_regime((n, r), regime, 29)
    if cfg == "gemv":
        force(path="gemv")
    elif cfg != "auto":
        force(path="gemm")
        force(tile=cfg)
    xb, x = acts(30, m, k)
    y = q2.q2_linear_lowrank(x, p[0], p[1], dev_bits(a, torch.float16), dev_bits(b, torch.float16)).cpu().numpy()
    ref = O.q2_linear_lowrank(xb, p_ref, s_ref, a, b)
    assert np.all(np.isfinite(y)) and np.any(ref != 0)
    assert_close(y, ref, f"low-rank branch alone, {regime} factors, {cfg} M={m} r={r}")


@pytest.mark.parametrize("m,n,k", [(65536, 64, 128), (1, 1 << 20, 128), (40, 300000, 256), (3000, 7, 384)])
def test_large_grids(m, n, k):
    """Far more workgroups than the benchmark shapes launch: many row tiles
    with few columns, 2^16 GEMV workgroups, 2^14 column tiles; Q2_0 and
    4-bit, sampled columns where N is large."""
    p_dev, s_dev, p_ref, s_ref = q2_weights(33, n, k)
    xb, x = acts(33, m, k)
    y = q2.q2_linear(x, p_dev, s_dev).cpu().numpy()
    cols = sample_cols(n, 256, seed=3) if n > 4096 else np.arange(n)
    assert_close(y[:, cols], O.q2_linear_cols(xb, p_ref, s_ref, cols), f"Q2_0 M={m} N={n} K={k}")
    p4, s4, z4, xb4, x4, P, S, Z = q4_case(34, m, k, n)
    y4 = q2.q4_linear(x4, P, S, Z).cpu().numpy()
    assert_close(y4[:, cols], O.q4_linear_cols(xb4, p4, s4, z4, cols), f"4-bit M={m} N={n} K={k}")
