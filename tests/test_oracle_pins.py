"""Pins of the CPU oracle to facts that do not come from the oracle itself:
hand-built examples derived from the pages' format definitions (tests/golden),
exhaustive decoding against the number formats' definitions, closed forms,
invariants the pages state, special cases that reduce to a library routine,
and exact rational brute force on tiny inputs.

The checks are written as functions of the implementation under test so that
test_planted_mistakes can run them against deliberately broken copies of the
oracle and show that each plausible mistake is caught.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.q2_oracle as O
from ternary_weight_quantized_q2_amd import inputs as I
from tests.conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vec = O.f16_to_f64(bits)
    hand = np.array([O.f16_decode_scalar(int(b)) for b in bits])
    nan = np.isnan(hand)
    assert np.array_equal(nan, np.isnan(vec))
    assert np.array_equal(hand[~nan], vec[~nan])
    # sign bits survive for zeros, and a few anchors of the binary16 definition
    assert math.copysign(1.0, O.f16_decode_scalar(0x8000)) == -1.0
    assert O.f16_decode_scalar(0x3C00) == 1.0
    assert O.f16_decode_scalar(0x7BFF) == 65504.0
    assert O.f16_decode_scalar(0x0001) == 2.0 ** -24
    assert O.f16_decode_scalar(0x0400) == 2.0 ** -14


def test_f16_cast_roundtrip_is_identity():
    # every non-NaN pattern -> float32 -> f16 must give the same pattern
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.f16_to_f64(bits).astype(np.float32)
    keep = ~np.isnan(vals)
    assert np.array_equal(I.f32_to_f16_bits(vals[keep]), bits[keep])


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vec = O.bf16_to_f64(bits)
    hand = np.array([O.bf16_decode_scalar(int(b)) for b in bits])
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(hand)
    assert np.array_equal(nan, np.isnan(vec)) and np.array_equal(nan, np.isnan(ref))
    assert np.array_equal(hand[~nan], vec[~nan])
    assert np.array_equal(ref[~nan], vec[~nan])


def test_fast_code_generator_distribution():
    """The digit-mapped generator of the layer lists draws codes in {0, 1, 2}
    with p = (0.3, 0.4, 0.3), reproducibly from its seed."""
    c = I.q2_codes_fast(97, 300, 1024)
    assert c.dtype == np.uint8 and c.shape == (300, 1024) and c.max() <= 2
    freq = np.bincount(c.ravel(), minlength=3) / c.size
    assert np.allclose(freq, [0.3, 0.4, 0.3], atol=0.005)
    assert np.array_equal(c, I.q2_codes_fast(97, 300, 1024))
    assert not np.array_equal(c, I.q2_codes_fast(98, 300, 1024))


def test_bf16_rounding_of_inputs_is_nearest_even():
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32)
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Q2_0 layout: the hand-built 2-byte example
# ---------------------------------------------------------------------------

def q2_bit_order_case():
    g = golden("q2_bit_order.json")
    k = g["K"]
    codes = np.full((1, k), g["codes_rest"], dtype=np.uint8)
    codes[0, :8] = g["codes_head"]
    x = np.zeros((1, k), dtype=np.float32)
    x[0, :8] = g["x_head"]
    xb = I.f32_to_bf16_bits(x)
    packed = np.full((1, k // 4), g["packed_rest"], dtype=np.uint8)
    packed[0, :2] = g["packed_head"]
    sc = np.full((1, 1), g["scale_f16_bits"], dtype=np.uint16)
    return g, codes, xb, packed, sc


def check_q2_bit_order(pack, unpack, linear):
    g, codes, xb, packed, sc = q2_bit_order_case()
    p, s = pack(codes, O.f16_to_f64(sc).astype(np.float32))
    assert np.array_equal(p, packed), "packer byte layout"
    assert np.array_equal(s, sc)
    w = unpack(packed, sc)
    assert np.array_equal(w, codes.astype(np.float64) - 1.0), "unpack layout"
    y = linear(xb, packed, sc)
    assert y.shape == (1, 1) and y[0, 0] == g["y"]


def test_q2_bit_order_golden():
    check_q2_bit_order(O.pack_q2, O.unpack_q2, O.q2_linear)


def test_q2_golden_discriminates_misreadings():
    # the two plausible misreadings of the layout give the fixture's other values
    g, codes, xb, packed, sc = q2_bit_order_case()
    x = O.bf16_to_f64(xb)[0]
    b = packed[0]
    msb = [((int(b[k // 4]) >> (6 - 2 * (k % 4))) & 3) - 1 for k in range(128)]
    strided = [((int(b[k % 32]) >> (2 * (k // 32))) & 3) - 1 for k in range(128)]
    assert float(np.dot(x, msb)) == g["y_if_msb_first"]
    assert float(np.dot(x, strided)) == g["y_if_strided_interleave"]
    assert g["y"] not in (g["y_if_msb_first"], g["y_if_strided_interleave"])


def test_unpack_scalar_equals_vectorised():
    codes = I.q2_codes(91, 5, 256)
    codes[0, :4] = 3  # the 2-bit field's fourth value decodes by the same formula
    sc = I.f32_to_f16_bits(I.q2_scales(91, 5, 256) * np.float32(-1.0) ** np.arange(10).reshape(5, 2))
    c = codes.reshape(5, 64, 4).astype(np.uint32)
    packed = (c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6).astype(np.uint8)
    lit = np.array(O.unpack_q2_scalar(packed, sc, 5, 256))
    assert np.array_equal(lit, O.unpack_q2(packed, sc))
    assert np.array_equal(O.codes_q2(packed), codes)


# ---------------------------------------------------------------------------
# Q2_0 closed forms
# ---------------------------------------------------------------------------

def check_q2_closed_forms(linear):
    m, k, n = 3, 384, 5
    xb = I.activations_bf16(92, m, k)
    x = O.bf16_to_f64(xb)
    ones = np.full((n, k // 4), 0x55, np.uint8)    # every code 1
    twos = np.full((n, k // 4), 0xAA, np.uint8)    # every code 2
    zeros = np.zeros((n, k // 4), np.uint8)        # every code 0
    sc_rand = I.f32_to_f16_bits(I.q2_scales(92, n, k))
    sc_one = np.full((n, k // 128), 0x3C00, np.uint16)
    sc_pow = np.tile(np.array([0x3C00, 0x4400, 0x3800], np.uint16), (n, 1))   # d = 1, 4, 0.5 per block
    assert np.all(linear(xb, ones, sc_rand) == 0.0)
    rs = x.sum(axis=1, keepdims=True)
    assert np.allclose(linear(xb, twos, sc_one), np.repeat(rs, n, 1), rtol=1e-14, atol=1e-12)
    assert np.allclose(linear(xb, zeros, sc_one), -np.repeat(rs, n, 1), rtol=1e-14, atol=1e-12)
    # per-block scale: code 2 in block 1 only, d = 4 there (1 and 0.5 elsewhere) -> 4 * sum over block 1
    w = np.full((n, k // 4), 0x55, np.uint8)
    w[:, 32:64] = 0xAA
    y = linear(xb, w, sc_pow)
    assert np.allclose(y, np.repeat(4.0 * x[:, 128:256].sum(1, keepdims=True), n, 1), rtol=1e-14, atol=1e-12)


def test_q2_closed_forms():
    check_q2_closed_forms(O.q2_linear)


# ---------------------------------------------------------------------------
# Q2_0 exact brute force and invariants
# ---------------------------------------------------------------------------

def check_q2_exact_bruteforce(linear, m=4, k=256, n=64, cfg=1):
    codes = I.q2_codes(cfg, n, k)
    sc = I.f32_to_f16_bits(I.q2_scales(cfg, n, k))
    xb = I.activations_bf16(cfg, m, k)
    c = codes.reshape(n, k // 4, 4).astype(np.uint32)
    packed = (c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6).astype(np.uint8)
    y = linear(xb, packed, sc)
    # exact rationals, from codes and scales directly (no oracle decoding)
    xs = [[Fraction(O.bf16_decode_scalar(int(v))) for v in row] for row in xb]
    ds = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in sc]
    for i in range(m):
        for j in range(n):
            terms = [xs[i][kk] * (int(codes[j, kk]) - 1) * ds[j][kk // 128] for kk in range(k)]
            exact = sum(terms, Fraction(0))
            bound = k * 2.0 ** -53 * float(sum(abs(t) for t in terms))
            assert abs(Fraction(float(y[i, j])) - exact) <= Fraction(bound) + Fraction(1, 2 ** 1074)


def test_q2_exact_bruteforce_tiny_config():
    check_q2_exact_bruteforce(O.q2_linear)


def test_row_slice_is_byte_range_slice():
    # rows are independent byte runs: y for W[n0:n1] is y[:, n0:n1]
    m, k, n = 3, 512, 40
    codes = I.q2_codes(93, n, k)
    packed, sc = O.pack_q2(codes, I.q2_scales(93, n, k))
    xb = I.activations_bf16(93, m, k)
    y = O.q2_linear(xb, packed, sc)
    flat = packed.reshape(-1)
    n0, n1 = 7, 29
    sub = flat[n0 * (k // 4):n1 * (k // 4)].reshape(n1 - n0, k // 4)
    ys = O.q2_linear(xb, sub, sc[n0:n1])
    assert np.allclose(ys, y[:, n0:n1], rtol=1e-13, atol=1e-13)
    assert np.allclose(O.q2_linear_cols(xb, packed, sc, np.arange(n0, n1)), y[:, n0:n1], rtol=1e-13, atol=1e-13)


def test_input_axis_split_is_sum_of_two_products():
    m, k, n, k1 = 4, 640, 24, 256
    codes = I.q2_codes(94, n, k)
    packed, sc = O.pack_q2(codes, I.q2_scales(94, n, k))
    xb = I.activations_bf16(94, m, k)
    y = O.q2_linear(xb, packed, sc)
    y1 = O.q2_linear(xb[:, :k1], packed[:, :k1 // 4], sc[:, :k1 // 128])
    y2 = O.q2_linear(xb[:, k1:], packed[:, k1 // 4:], sc[:, k1 // 128:])
    assert np.allclose(y1 + y2, y, rtol=1e-12, atol=1e-12)


SLICE_CASES = [(0, 9, 0, 640), (2, 7, 128, 384), (8, 9, 512, 640), (0, 1, 0, 128), (3, 3, 0, 128),
               (4, 6, 256, 256), (1, 8, 384, 640)]


def check_slice(slice_fn):
    """A slice decodes, element by element, to the matching part of the whole
    matrix under the literal per-element decode (pinned by the bit-order and
    closed-form checks), and its bytes are those of the sliced codes packed
    afresh."""
    n, k = 9, 640
    codes = I.q2_codes(97, n, k)
    scales = I.q2_scales(97, n, k)
    packed, sc = O.pack_q2(codes, scales)
    full = O.unpack_q2_scalar(packed, sc, n, k)
    for n0, n1, k0, k1 in SLICE_CASES:
        sp, ss = slice_fn(packed, sc, n0, n1, k0, k1)
        assert sp.shape == (n1 - n0, (k1 - k0) // 4) and ss.shape == (n1 - n0, (k1 - k0) // 128)
        if n1 > n0 and k1 > k0:
            assert O.unpack_q2_scalar(sp, ss, n1 - n0, k1 - k0) == [row[k0:k1] for row in full[n0:n1]]
            want_p, want_s = O.pack_q2(codes[n0:n1, k0:k1], scales[n0:n1, k0 // 128:k1 // 128])
            assert np.array_equal(sp, want_p) and np.array_equal(ss, want_s)


def test_slice_pins():
    check_slice(O.slice_q2)
    with pytest.raises(ValueError):
        O.slice_q2(np.zeros((2, 64), np.uint8), np.zeros((2, 2), np.uint16), 0, 2, 64, 256)


def check_split_sum(sum_fn):
    """The fused output projection computed as two products over input slices
    (low-rank A sliced the same way, B shared) plus an existing y0 equals y0
    plus the whole product, against exact rationals built from the codes."""
    m, k, n, k1, r = 2, 384, 5, 128, 3
    codes = I.q2_codes(98, n, k)
    packed, sc = O.pack_q2(codes, I.q2_scales(98, n, k))
    xb = I.activations_bf16(98, m, k)
    a, b = I.lowrank_factors(98, r, k, n, std=0.1)
    y0 = np.random.default_rng(98).standard_normal((m, n))
    parts = [(np.ascontiguousarray(xb[:, :k1]), np.ascontiguousarray(packed[:, :k1 // 4]),
              np.ascontiguousarray(sc[:, :k1 // 128]), np.ascontiguousarray(a[:, :k1]), b),
             (np.ascontiguousarray(xb[:, k1:]), np.ascontiguousarray(packed[:, k1 // 4:]),
              np.ascontiguousarray(sc[:, k1 // 128:]), np.ascontiguousarray(a[:, k1:]), b)]
    y = sum_fn(parts, y0)
    xs = [[Fraction(O.bf16_decode_scalar(int(v))) for v in row] for row in xb]
    ds = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in sc]
    av = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in a]
    bv = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in b]
    for i in range(m):
        t = [sum((xs[i][kk] * av[j][kk] for kk in range(k)), Fraction(0)) for j in range(r)]
        for j in range(n):
            w = sum((xs[i][kk] * (int(codes[j, kk]) - 1) * ds[j][kk // 128] for kk in range(k)), Fraction(0))
            exact = Fraction(float(y0[i, j])) + w + sum((t[q] * bv[j][q] for q in range(r)), Fraction(0))
            assert abs(float(Fraction(float(y[i, j])) - exact)) <= 1e-12 * (1.0 + abs(float(exact)))
    # without y0 the sum starts from the first part
    assert np.array_equal(sum_fn(parts[:1]), O.q2_linear_lowrank(*parts[0]))


def test_split_sum_pins():
    check_split_sum(O.q2_linear_sum)


def _expect_import_error(call, kind, index):
    try:
        call()
    except O.ImportError_ as e:
        assert (e.kind, e.index) == (kind, index), (e.kind, e.index)
        return
    raise AssertionError(f"conversion did not stop on the bad {kind}")


def _source_codes_literal(ct):
    """Codes [N, K] of a transposed source, one 2-bit field at a time."""
    kq, n = ct.shape
    out = np.zeros((n, 4 * kq), np.uint8)
    for j in range(kq):
        for i in range(4):
            out[:, 4 * j + i] = (ct[j, :] >> (2 * i)) & 3
    return out


def check_import(import_fn):
    g = golden("import_transpose.json")
    k, n = g["K"], g["N"]
    ct = np.full((k // 4, n), g["source_rest"], np.uint8)
    ct[:len(g["source_col0_head"]), 0] = g["source_col0_head"]
    ct[:len(g["source_col1_head"]), 1] = g["source_col1_head"]
    st = np.array([g["scales"]], np.float32)
    zt = np.array([g["zeros"]], np.float32)
    p, s = import_fn(ct, st, zt, g["G"])
    assert list(p[0, :2]) == g["packed_row0_head"] and list(p[1, :3]) == g["packed_row1_head"]
    assert list(s[:, 0]) == g["scale_f16_bits"]
    w = O.unpack_q2(p, s)
    assert list(w[0, :8]) == g["w_row0_head"] and list(w[1, :8]) == g["w_row1_head"]
    # no numeric change: the Q2_0 weight equals the source's own dequantisation, element by element
    for group in (32, 64, 128, 256):
        n2, k2 = 37, 512
        ct2, st2, zt2 = I.gemlite_source(group, n2, k2, group)
        p2, s2 = import_fn(ct2, st2, zt2, group)
        assert np.array_equal(O.unpack_q2(p2, s2), O.gemlite_dequant(ct2, st2, zt2, group)), group
        # and, independently of both oracle decoders: the codes read field by
        # field from the source bytes (byte j of column n holds codes 4j..4j+3
        # of row n, least significant pair first), and each block's scale is
        # the source scale of the group holding the block's first weight
        assert np.array_equal(O.codes_q2(p2), _source_codes_literal(ct2)), group
        first_group = (np.arange(k2 // 128) * 128) // group
        assert np.array_equal(np.asarray(s2).view(np.float16).astype(np.float32), st2[first_group, :].T), group
    # the conversion stops, naming the first offending element, in the order codes, zeros, scales
    ct2, st2, zt2 = I.gemlite_source(7, 6, 256, 64)
    bad = ct2.copy()
    bad[5, 3] |= 0x30                                   # weight row 3, k = 4 * 5 + 2 becomes code 3
    _expect_import_error(lambda: import_fn(bad, st2, zt2, 64), "code", 3 * 256 + 22)
    z = zt2.copy()
    z[2, 4] = -z[2, 4]                                  # zero == +scale
    _expect_import_error(lambda: import_fn(ct2, st2, z, 64), "zero", 2 * 6 + 4)
    sc = st2.copy()
    sc[1, 1] = np.float32(0.1)                          # not an f16 value (zero kept equal to -scale)
    _expect_import_error(lambda: import_fn(ct2, sc, -sc, 64), "scale", 1 * 6 + 1)
    sc2 = st2.copy()
    sc2[3, 5] = sc2[3, 5] * 2                            # second group of block 1 disagrees with the first
    _expect_import_error(lambda: import_fn(ct2, sc2, -sc2, 64), "scale", 3 * 6 + 5)


def test_import_pins():
    check_import(O.import_gemlite)
    with pytest.raises(ValueError):
        O.import_gemlite(np.zeros((32, 2), np.uint8), np.zeros((3, 2), np.float32), np.zeros((3, 2), np.float32), 48)


def check_a8(quantize, linear_a8):
    """8-bit activations: the hand-built row; every code within half a step of
    x / s; the row maximum at +-127; one scale per row; a zero row; and the
    product within the quantisation bound of the unquantised one."""
    g = golden("a8_hand.json")
    k = g["K"]
    x = np.zeros((1, k), np.float32)
    x[0, :len(g["x_head"])] = g["x_head"]
    xb = I.f32_to_bf16_bits(x)
    q, sc = quantize(xb)
    assert list(q[0, :8]) == g["codes_head"] and not q[0, 8:].any()
    assert int(np.asarray(sc, np.float32).view(np.uint32)[0]) == g["scale_f32_bits"]
    codes = np.ones((1, k), np.uint8)
    codes[0, :8] = g["w_codes_head"]
    packed, scb = O.pack_q2(codes, np.ones((1, 1), np.float32))
    y = linear_a8(xb, packed, scb)
    s = float(np.asarray(sc, np.float32)[0])
    assert y[0, 0] == g["code_sum"] * s
    assert abs(y[0, 0] - g["y_unquantized"]) < 0.01 * g["y_unquantized"]
    # random rows of different ranges, one of them all zeros
    m, k2, n = 5, 384, 9
    xr = I.activations_bf16(99, m, k2).copy()
    xf = (xr.astype(np.uint32) << 16).view(np.float32).copy()
    xf[1] *= 64.0
    xf[3] = 0.0
    xr = I.f32_to_bf16_bits(xf)
    xf = (xr.astype(np.uint32) << 16).view(np.float32)
    q, sc = quantize(xr)
    sc = np.asarray(sc, np.float32)
    amax = np.abs(xf).max(axis=1)
    assert sc[3] == 0 and not q[3].any()
    for r in (0, 1, 2, 4):
        assert abs(float(sc[r]) - float(amax[r]) / 127) <= 2.0 ** -23 * float(amax[r]) / 127
        assert np.abs(q[r]).max() == 127
        err = np.abs(xf[r].astype(np.float64) / float(sc[r]) - q[r])
        assert err.max() <= 0.5 + 1e-5
    assert abs(float(sc[1]) / float(sc[0]) - float(amax[1]) / float(amax[0])) < 1e-6 * float(sc[1] / sc[0])
    codes = I.q2_codes(99, n, k2)
    packed, scb = O.pack_q2(codes, I.q2_scales(99, n, k2))
    w = O.unpack_q2(packed, scb)
    ya8 = linear_a8(xr, packed, scb)
    yref = O.q2_linear(xr, packed, scb)
    bound = (sc.astype(np.float64)[:, None] / 2) * (np.abs(w).sum(axis=1)[None, :]) * (1 + 1e-5)
    assert np.all(np.abs(ya8 - yref) <= bound)
    assert not ya8[3].any()


def test_a8_pins():
    check_a8(O.quantize_rows_a8, O.q2_linear_a8)


# ---------------------------------------------------------------------------
# pack: scale round trip and code check
# ---------------------------------------------------------------------------

def test_pack_scale_roundtrip_rules():
    g = golden("pack_scales.json")
    codes = np.ones((1, 128), np.uint8)
    for v in g["accept"]:
        _, s = O.pack_q2(codes, np.array([[v]], np.float32))
        assert O.f16_to_f64(s)[0, 0] == np.float32(v)
    for v in g["reject"]:
        with pytest.raises(O.PackError) as e:
            O.pack_q2(codes, np.array([[float(v)]], np.float32))
        assert e.value.kind == "scale" and e.value.index == 0


def test_pack_reports_first_bad_index_codes_before_scales():
    codes = np.ones((3, 256), np.uint8)
    sc = np.ones((3, 2), np.float32)
    codes[1, 200] = 3
    codes[2, 5] = 7
    sc[0, 1] = 1.000244140625
    with pytest.raises(O.PackError) as e:
        O.pack_q2(codes, sc)
    assert e.value.kind == "code" and e.value.index == 256 + 200
    codes[:] = 2
    with pytest.raises(O.PackError) as e:
        O.pack_q2(codes, sc)
    assert e.value.kind == "scale" and e.value.index == 1


# ---------------------------------------------------------------------------
# low-rank branch
# ---------------------------------------------------------------------------

def lowrank_hand_case():
    g = golden("lowrank_hand.json")
    k, n, r = g["K"], g["N"], g["r"]
    a = np.zeros((r, k), np.float32)
    for i, j, v in g["A_entries"]:
        a[i, j] = v
    x = np.zeros((1, k), np.float32)
    x[0, :len(g["x_head"])] = g["x_head"]
    packed = np.full((n, k // 4), 0x55, np.uint8)
    sc = I.f32_to_f16_bits(np.full((n, 1), 0.75, np.float32))
    return (g, I.f32_to_bf16_bits(x), packed, sc, I.f32_to_f16_bits(a),
            I.f32_to_f16_bits(np.array(g["B"], np.float32)))


def check_lowrank(lowrank):
    g, xb, packed, sc, a, b = lowrank_hand_case()
    y = lowrank(xb, packed, sc, a, b)
    assert np.array_equal(y[0], np.array(g["y"], np.float64))
    # r = 0 is the plain linear; associativity: B (A x) == (B A) x
    m, k, n, r = 3, 384, 20, 6
    codes = I.q2_codes(95, n, k)
    packed, sc = O.pack_q2(codes, I.q2_scales(95, n, k))
    xb = I.activations_bf16(95, m, k)
    a, b = I.lowrank_factors(95, r, k, n, std=0.1)
    empty_a = np.zeros((0, k), np.uint16)
    empty_b = np.zeros((n, 0), np.uint16)
    assert np.array_equal(lowrank(xb, packed, sc, empty_a, empty_b), O.q2_linear(xb, packed, sc))
    ba = O.f16_to_f64(b) @ O.f16_to_f64(a)            # [n, k]
    ref = O.bf16_to_f64(xb) @ (O.unpack_q2(packed, sc) + ba).T
    assert np.allclose(lowrank(xb, packed, sc, a, b), ref, rtol=1e-12, atol=1e-13)


def test_lowrank_pins():
    check_lowrank(O.q2_linear_lowrank)


def test_lowrank_hand_discriminates_transpose():
    g, xb, packed, sc, a, b = lowrank_hand_case()
    t = O.bf16_to_f64(xb) @ O.f16_to_f64(a).T
    assert np.array_equal((t @ O.f16_to_f64(b))[0], np.array(g["y_if_B_transposed"], np.float64))


def test_lowrank_exact_bruteforce():
    m, k, n, r = 2, 256, 6, 3
    codes = I.q2_codes(96, n, k)
    packed, sc = O.pack_q2(codes, I.q2_scales(96, n, k))
    xb = I.activations_bf16(96, m, k)
    a, b = I.lowrank_factors(96, r, k, n)
    y = O.q2_linear_lowrank(xb, packed, sc, a, b)
    X = [[Fraction(O.bf16_decode_scalar(int(v))) for v in row] for row in xb]
    A = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in a]
    B = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in b]
    D = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in sc]
    for i in range(m):
        t = [sum((X[i][kk] * A[j][kk] for kk in range(k)), Fraction(0)) for j in range(r)]
        for nn in range(n):
            exact = sum((X[i][kk] * (int(codes[nn, kk]) - 1) * D[nn][kk // 128] for kk in range(k)), Fraction(0))
            exact += sum((B[nn][j] * t[j] for j in range(r)), Fraction(0))
            assert abs(float(y[i, nn]) - float(exact)) <= 1e-13 * (1 + abs(float(exact)))


# ---------------------------------------------------------------------------
# 4-bit nibble variant
# ---------------------------------------------------------------------------

def q4_hand_case():
    g = golden("q4_nibble_order.json")
    k = g["K"]
    p4 = np.zeros((1, k // 2), np.uint8)
    p4[0, :2] = g["bytes_head"]
    x = np.zeros((1, k), np.float32)
    x[0, :4] = g["x_head"]
    s = np.full((1, 1), g["scale_f16_bits"], np.uint16)
    z = np.full((1, 1), g["zero_f16_bits"], np.uint16)
    return g, I.f32_to_bf16_bits(x), p4, s, z


def check_q4(q4_linear):
    g, xb, p4, s, z = q4_hand_case()
    assert q4_linear(xb, p4, s, z)[0, 0] == g["y"]
    # scale 1, zero 0: W is the integer code matrix, y = X @ codes^T (library matmul)
    m, k, n = 3, 256, 7
    p4, _, _ = I.q4_weights(97, n, k)
    xb = I.activations_bf16(97, m, k)
    one = np.full((n, 2), 0x3C00, np.uint16)
    zero = np.zeros((n, 2), np.uint16)
    lo = (p4 & 15).astype(np.float64)
    hi = (p4 >> 4).astype(np.float64)
    codes = np.stack([lo, hi], axis=-1).reshape(n, k)
    assert np.allclose(q4_linear(xb, p4, one, zero), O.bf16_to_f64(xb) @ codes.T, rtol=1e-13, atol=1e-12)
    # every code equal to an integer zero point -> y = 0 exactly
    same = np.full((n, k // 2), 0x77, np.uint8)
    seven = I.f32_to_f16_bits(np.full((n, 2), 7.0, np.float32))
    assert np.all(q4_linear(xb, same, I.q4_weights(98, n, k)[1], seven) == 0.0)


def test_q4_pins():
    check_q4(O.q4_linear)


def check_q4_cols(cols_fn):
    """The sampled-column 4-bit product equals the columns of the whole
    (pinned) 4-bit product, for single, scattered, repeated-order and all
    columns, with zero points that are not integers."""
    m, k, n = 3, 384, 29
    p4, s, z = I.q4_weights(96, n, k)
    xb = I.activations_bf16(96, m, k)
    full = O.q4_linear(xb, p4, s, z)
    for cols in (np.array([0]), np.array([n - 1]), np.array([17, 2, 9]), np.arange(n)):
        got = cols_fn(xb, p4, s, z, cols)
        assert got.shape == (m, len(cols))
        assert np.allclose(got, full[:, cols], rtol=1e-13, atol=1e-13), cols


def test_q4_cols_pins():
    check_q4_cols(O.q4_linear_cols)


def test_q4_exact_bruteforce():
    m, k, n = 2, 256, 5
    p4, s, z = I.q4_weights(99, n, k)
    xb = I.activations_bf16(99, m, k)
    y = O.q4_linear(xb, p4, s, z)
    X = [[Fraction(O.bf16_decode_scalar(int(v))) for v in row] for row in xb]
    S = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in s]
    Z = [[Fraction(O.f16_decode_scalar(int(v))) for v in row] for row in z]
    for i in range(m):
        for nn in range(n):
            terms = []
            for kk in range(k):
                byte = int(p4[nn, kk // 2])
                q = (byte >> 4) if kk % 2 else (byte & 15)
                terms.append(X[i][kk] * (q - Z[nn][kk // 128]) * S[nn][kk // 128])
            exact = sum(terms, Fraction(0))
            bound = k * 2.0 ** -52 * float(sum(abs(t) for t in terms))
            assert abs(Fraction(float(y[i, nn])) - exact) <= Fraction(bound) + Fraction(1, 2 ** 1074)


# ---------------------------------------------------------------------------
# acceptance rule
# ---------------------------------------------------------------------------

def test_acceptance_rule():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((8, 300))
    assert O.acceptance(ref, ref)["ok"]
    assert O.acceptance(ref * (1 + 5e-5), ref)["ok"]
    assert not O.acceptance(ref * (1 + 2e-4), ref)["ok"]            # relative L2 too large
    spike = ref.copy()
    spike[3, 17] += 2e-3 * np.sqrt(np.mean(ref[3] ** 2))              # one element, 2e-3 of its row RMS
    r = O.acceptance(spike, ref)
    assert r["rel_l2"] < 1e-4 and not r["ok"]
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert not O.acceptance(bad, ref)["ok"]
    z = np.zeros((2, 5))
    assert O.acceptance(z, z)["ok"] and not O.acceptance(z + 1e-30, z)["ok"]
