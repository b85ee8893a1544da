"""GPU parity of weight slicing and of the input-axis split with accumulation
(q2_slice, q2_linear_ex with Q2_ACCUMULATE) against the CPU oracle.

Bars: slices bit-exact (codes and scale bits); an accumulating call gives,
bit for bit, y0 + v in fp32 where v is what the same call writes without the
flag; the split product within the linear's tolerance of the oracle's whole
product.
"""
import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
import ternary_weight_quantized_q2_amd as q2
from ternary_weight_quantized_q2_amd import inputs as I
from tests.test_parity_gpu import DEV, acts, assert_close, dev_bits, host_bits, q2_weights, sample_cols

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU; they must not be skipped silently"
    torch.cuda.set_device(0)
    q2.load()
    yield


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------

SLICES = [(0, 9, 0, 640), (2, 7, 128, 384), (8, 9, 512, 640), (0, 1, 0, 128), (3, 3, 0, 128), (4, 6, 256, 256),
          (1, 8, 384, 640)]


@pytest.mark.parametrize("n0,n1,k0,k1", SLICES)
def test_slice_bitexact(n0, n1, k0, k1):
    p_dev, s_dev, p_ref, s_ref = q2_weights(41, 9, 640)
    sp, ss = q2.q2_slice(p_dev, s_dev, n0, n1, k0, k1)
    torch.cuda.synchronize()
    want_p, want_s = O.slice_q2(p_ref, s_ref, n0, n1, k0, k1)
    assert np.array_equal(sp.cpu().numpy(), want_p)
    assert np.array_equal(host_bits(ss), want_s)


# Fused projection of a transformer block at hidden size 3072: Q, K, V and the
# MLP input (4 x 3072) as one weight of 21504 rows.
FUSED_PARTS = [(0, 3072), (3072, 6144), (6144, 9216), (9216, 21504)]


def test_fused_weight_row_slices():
    n, k, m = 21504, 3072, 96
    p_dev, s_dev, p_ref, s_ref = q2_weights(42, n, k)
    xb, x = acts(42, m, k)
    for n0, n1 in FUSED_PARTS:
        sp, ss = q2.q2_slice(p_dev, s_dev, n0, n1, 0, k)
        torch.cuda.synchronize()
        want_p, want_s = O.slice_q2(p_ref, s_ref, n0, n1, 0, k)
        assert np.array_equal(sp.cpu().numpy(), want_p), (n0, n1)
        assert np.array_equal(host_bits(ss), want_s), (n0, n1)
        # a row range is also usable in place: rows are contiguous byte runs
        y_copy = q2.q2_linear(x, sp, ss)
        y_view = q2.q2_linear(x, p_dev[n0:n1], s_dev[n0:n1])
        torch.cuda.synchronize()
        assert torch.equal(y_copy, y_view)
        cols = sample_cols(n1 - n0, 96, seed=n0)
        ref = O.q2_linear_cols(xb, want_p, want_s, cols)
        assert_close(y_copy.cpu().numpy()[:, cols], ref, f"fused rows [{n0}, {n1})")


def test_slice_errors():
    p_dev, s_dev, _, _ = q2_weights(43, 4, 256)
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_slice(p_dev, s_dev, 0, 4, 64, 256)
    assert e.value.status == q2.Q2_ERR_SHAPE
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_slice(p_dev, s_dev, 0, 5, 0, 256)
    assert e.value.status == q2.Q2_ERR_ARG


# ---------------------------------------------------------------------------
# accumulation: y0 + v, bit for bit, on every kernel configuration
# ---------------------------------------------------------------------------

GEMM_CFGS = ["w48x192", "w96x192", "w64x128", "w32x128", "w32x64",
             "kg2x1x4", "kg4x2x2", "kg2x1x2", "kg2x2x4", "kg2x2x2", "kg2x1x4r3", "kg6x3x2"]
LR_CFGS = ["kg6x3x2", "w48x192", "w96x192", "w64x128", "w32x128", "w32x64"]


def _set_path(force, cfg):
    force(path=None)
    force(tile=None)
    if cfg == "gemv":
        force(path="gemv")
    elif cfg != "auto":
        force(path="gemm")
        force(tile=cfg)


def _acc_case(cfg, m, n, k, r, unaligned=False):
    p, s, _, _ = q2_weights(44, n, k)
    _, x = acts(44, m, k)
    A = B = None
    if r:
        a, b = I.lowrank_factors(44, r, k, n, std=0.02)
        A, B = dev_bits(a, torch.float16), dev_bits(b, torch.float16)
    g = torch.Generator().manual_seed(45)
    y0 = torch.randn((m, n), generator=g).to(DEV)
    if unaligned:                       # y 4 bytes past a 16-byte boundary: the per-element stores
        flat = torch.zeros(m * n + 4, device=DEV)
        y = flat[1:1 + m * n].view(m, n)
        assert y.data_ptr() % 16 == 4
        y.copy_(y0)
    else:
        y = y0.clone()
    v = q2.q2_linear_ex(x, p, s, A=A, B=B)
    q2.q2_linear_ex(x, p, s, y=y, A=A, B=B, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y0 + v), f"{cfg} M={m} N={n} K={k} r={r}"


@pytest.mark.parametrize("cfg", ["auto", "gemv"] + GEMM_CFGS)
def test_accumulate_is_y0_plus_result(cfg, force):
    _set_path(force, cfg)
    if cfg == "gemv":
        _acc_case(cfg, 5, 333, 640, 0)
        _acc_case(cfg, 16, 400, 1280, 0)
    else:
        _acc_case(cfg, 192, 400, 640, 0)                   # row-contiguous stores
        _acc_case(cfg, 192, 333, 640, 0)                   # N not a multiple of 4: per-element stores
        _acc_case(cfg, 192, 400, 640, 0, unaligned=True)


@pytest.mark.parametrize("cfg", ["auto", "gemv"] + LR_CFGS)
def test_accumulate_lowrank(cfg, force):
    _set_path(force, cfg)
    if cfg == "gemv":
        _acc_case(cfg, 3, 300, 384, 32)
    else:
        _acc_case(cfg, 192, 400, 640, 32)
        _acc_case(cfg, 192, 333, 640, 8)
        _acc_case(cfg, 192, 400, 640, 5)                   # a rank off the 8-multiple


def test_accumulate_empty_sum_keeps_y():
    m, n = 7, 40
    y0 = torch.randn((m, n), device=DEV)
    y = y0.clone()
    x = torch.empty((m, 0), dtype=torch.bfloat16, device=DEV)
    p = torch.empty((n, 0), dtype=torch.uint8, device=DEV)
    s = torch.empty((n, 0), dtype=torch.float16, device=DEV)
    q2.q2_linear_ex(x, p, s, y=y, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert torch.equal(q2.q2_linear_ex(x, p, s), torch.zeros_like(y0))


# ---------------------------------------------------------------------------
# the fused output projection as two products over input slices, summed
# ---------------------------------------------------------------------------

def _split(m, n, k1, k2, r, cols=None):
    k = k1 + k2
    p, s, p_ref, s_ref = q2_weights(46, n, k)
    xb, _ = acts(46, m, k)
    x1 = dev_bits(np.ascontiguousarray(xb[:, :k1]), torch.bfloat16)
    x2 = dev_bits(np.ascontiguousarray(xb[:, k1:]), torch.bfloat16)
    p1, s1 = q2.q2_slice(p, s, 0, n, 0, k1)
    p2, s2 = q2.q2_slice(p, s, 0, n, k1, k)
    A1 = A2 = B = None
    if r:
        a, b = I.lowrank_factors(46, r, k, n, std=0.02)
        A1 = dev_bits(np.ascontiguousarray(a[:, :k1]), torch.float16)
        A2 = dev_bits(np.ascontiguousarray(a[:, k1:]), torch.float16)
        B = dev_bits(b, torch.float16)
    y = q2.q2_linear_ex(x1, p1, s1, A=A1, B=B)
    q2.q2_linear_ex(x2, p2, s2, y=y, A=A2, B=B, accumulate=True)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    if cols is None:
        ref = O.q2_linear_lowrank(xb, p_ref, s_ref, a, b) if r else O.q2_linear(xb, p_ref, s_ref)
    else:
        ref = O.q2_linear_cols(xb, p_ref, s_ref, cols)
        if r:
            ref = ref + O.lowrank_t(xb, a) @ O.f16_to_f64(b[cols]).T
        y = y[:, cols]
    assert_close(y, ref, f"split M={m} N={n} K={k1}+{k2} r={r}")


@pytest.mark.parametrize("m", [1, 5, 75, 200])
@pytest.mark.parametrize("r", [0, 32])
def test_split_projection(m, r):
    _split(m, 333, 256, 384, r)


@pytest.mark.parametrize("r", [0, 32])
def test_split_projection_full_size(r):
    # single-block output projection: attention output (3072) and MLP output (12288) side by side
    _split(1536, 3072, 3072, 12288, r, cols=sample_cols(3072, 128, seed=7))


# ---------------------------------------------------------------------------
# import of a transposed group-quantised ternary weight
# ---------------------------------------------------------------------------

def _import_dev(ct, st, zt, group):
    return q2.q2_import_gemlite(torch.from_numpy(ct).to(DEV), torch.from_numpy(st).to(DEV),
                                torch.from_numpy(zt).to(DEV), group)


@pytest.mark.parametrize("n,k,group", [(37, 512, 32), (64, 1280, 64), (1000, 384, 128), (300, 1024, 256),
                                       (3, 1536, 512), (3072, 12288, 64)])
def test_import_bitexact(n, k, group):
    ct, st, zt = I.gemlite_source(group + n, n, k, group)
    p, s = _import_dev(ct, st, zt, group)
    torch.cuda.synchronize()
    want_p, want_s = O.import_gemlite(ct, st, zt, group)
    assert np.array_equal(p.cpu().numpy(), want_p)
    assert np.array_equal(host_bits(s), want_s)


def test_import_errors_match_the_oracle():
    n, k, group = 6, 256, 64
    ct, st, zt = I.gemlite_source(7, n, k, group)
    cases = []
    bad = ct.copy()
    bad[5, 3] |= 0x30
    bad[9, 1] |= 0x03                                  # a second code 3: the smaller weight index is reported
    cases.append((bad, st, zt, q2.Q2_ERR_CODE))
    z = zt.copy()
    z[2, 4] = -z[2, 4]
    z[3, 0] = 1.0
    cases.append((ct, st, z, q2.Q2_ERR_FORMAT))
    sc = st.copy()
    sc[1, 1] = np.float32(0.1)
    cases.append((ct, sc, -sc, q2.Q2_ERR_SCALE))
    sc2 = st.copy()
    sc2[3, 5] *= 2
    cases.append((ct, sc2, -sc2, q2.Q2_ERR_SCALE))
    both = bad.copy()
    cases.append((both, sc, z, q2.Q2_ERR_CODE))            # codes are checked first
    for ct_, st_, zt_, status in cases:
        with pytest.raises(O.ImportError_) as ref:
            O.import_gemlite(ct_, st_, zt_, group)
        with pytest.raises(q2.Q2Error) as e:
            _import_dev(ct_, st_, zt_, group)
        assert e.value.status == status
        assert e.value.bad_index == ref.value.index


# ---------------------------------------------------------------------------
# every entry point runs on the caller's stream
# ---------------------------------------------------------------------------

def test_calls_run_on_the_callers_stream():
    """A side stream is kept busy, then the input is written on it and each
    entry point is called on it: a launch on any other stream would read the
    input before it is written.  Results equal the same calls on the default
    stream, bit for bit (every call is deterministic)."""
    k, n = 1280, 333
    p, s, _, _ = q2_weights(47, n, k)
    p4, s4, z4 = I.q4_weights(47, n, k)
    P4 = torch.from_numpy(p4).to(DEV)
    S4, Z4 = dev_bits(s4, torch.float16), dev_bits(z4, torch.float16)
    a, b = I.lowrank_factors(47, 32, k, n, std=0.02)
    A, B = dev_bits(a, torch.float16), dev_bits(b, torch.float16)
    calls = {
        "gemm": lambda x: q2.q2_linear(x, p, s),
        "lowrank": lambda x: q2.q2_linear_lowrank(x, p, s, A, B),
        "q4": lambda x: q2.q4_linear(x, P4, S4, Z4),
        "a8": lambda x: q2.q2_linear_a8(x, p, s),
        "accumulate": lambda x: q2.q2_linear_ex(x, p, s, y=torch.ones((x.shape[0], n), device=DEV), accumulate=True),
    }
    side = torch.cuda.Stream()
    for m in (200, 5):                                   # the GEMM and the GEMV paths
        _, x = acts(48, m, k)
        refs = {name: fn(x) for name, fn in calls.items()}
        torch.cuda.synchronize()
        for name, fn in calls.items():
            x_late = torch.zeros_like(x)
            busy = torch.randn(2048, 2048, device=DEV)
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                for _ in range(30):
                    busy = (busy @ busy) * 1e-3
                x_late.copy_(x)
                y = fn(x_late)
            side.synchronize()
            assert torch.equal(y, refs[name]), f"{name} M={m}"


# ---------------------------------------------------------------------------
# captured in a HIP graph, replayed with eager work in between
# ---------------------------------------------------------------------------

def test_graph_replays_match_eager():
    """Each entry point is captured once into a graph (static input, output
    and workspace buffers) and replayed three times; before each replay new
    activations are written eagerly, and after it the replay's output must
    equal an eager call on the same input, bit for bit.  The split case
    captures the zero fill and the two atomic parts of the K split."""
    def q2w(cfg, n, k):
        p, s, _, _ = q2_weights(cfg, n, k)
        return p, s

    cases = []
    p, s = q2w(51, 384, 12288)                          # long K over few tiles: K split
    cases.append(("split", 128, 12288, 384, lambda x, y, ws: q2.q2_linear(x, p, s, y), 0))
    p2, s2 = q2w(52, 333, 1280)
    cases.append(("gemm", 200, 1280, 333, lambda x, y, ws: q2.q2_linear(x, p2, s2, y), 0))
    cases.append(("gemv", 3, 1280, 333, lambda x, y, ws: q2.q2_linear(x, p2, s2, y), 0))
    a, b = I.lowrank_factors(53, 32, 1280, 333, std=0.02)
    A, B = dev_bits(a, torch.float16), dev_bits(b, torch.float16)
    cases.append(("lowrank", 192, 1280, 333,
                  lambda x, y, ws: q2.q2_linear_lowrank(x, p2, s2, A, B, y=y, workspace=ws),
                  q2.lowrank_workspace_bytes(192, 32)))
    cases.append(("a8", 100, 1280, 333, lambda x, y, ws: q2.q2_linear_a8(x, p2, s2, y=y, workspace=ws),
                  q2.a8_workspace_bytes(100, 1280)))
    cases.append(("a8 split", 64, 12288, 384, lambda x, y, ws: q2.q2_linear_a8(x, p, s, y=y, workspace=ws),
                  q2.a8_workspace_bytes(64, 12288)))
    p4, s4, z4 = I.q4_weights(54, 333, 1280)
    P4, S4, Z4 = torch.from_numpy(p4).to(DEV), dev_bits(s4, torch.float16), dev_bits(z4, torch.float16)
    cases.append(("q4", 64, 1280, 333, lambda x, y, ws: q2.q4_linear(x, P4, S4, Z4, y), 0))

    for name, m, k, n, fn, wsb in cases:
        x = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
        y = torch.empty((m, n), device=DEV)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
        _, x0 = acts(55, m, k)
        x.copy_(x0)
        fn(x, y, ws)                                       # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(x, y, ws)
        torch.cuda.synchronize()
        y_e = torch.empty_like(y)
        ws_e = torch.empty_like(ws)
        for rep in range(3):
            _, xr = acts(56 + rep, m, k)
            x.copy_(xr)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            fn(x, y_e, ws_e)
            torch.cuda.synchronize()
            assert torch.equal(y, y_e), f"{name} replay {rep}"
