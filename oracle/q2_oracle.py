"""CPU oracle for the Q2_0 ternary linear, its low-rank side branch and the
4-bit nibble variant.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
definition of what the HIP library computes.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the library and
its Python binding never do, and the two share no code.

Everything is NumPy float64 (or exact Python integers in the scalar
helpers).  Every decoded value below is exact in float64: bf16 and f16 values
are exact, a bf16 x f16 product has at most 8 + 11 significant bits, and the
4-bit dequantised weight (q - z) * s is computed exactly from f16 inputs.  The
only rounding is float64 summation inside a BLAS dgemm, far below the 1e-4
relative tolerance the GPU path is held to.

Sources (web pages on ternary-weight image models):
* "We're Teaching Your Browser to Paint" (aitherium.com), section "The lucky
  break that wasn't luck": codes {0,1,2} packed LSB-first four per byte along
  the input axis; 128-weight blocks with one f16 scale; a weight is (q - 1) x d;
  the converter's only rounding is the f32 -> f16 scale cast and it aborts when
  that cast is not exact.
* same page, section "The GPU driver...": 2-bit rows are independent byte runs,
  so a row slice of the weight is a byte-range slice; a projection can be split
  along its input axis into two products that are summed.
* "You Can Now Just Ask for an Image" (aitherium.com), section "The bug that
  hid in one flipped bit": two 4-bit codes per byte, the low nibble holding the
  even position; and "We're Teaching..." section "What's left": the 4-bit
  encoder weights dequantise as (q - zero) x scale.
* mindview-t2i-turbo model card, section "One step": the side branch is
  y = W x + B (A x).

Readings where the pages leave a step open: consecutive codes share a byte
(code k sits in bits 2(k%4)..2(k%4)+1 of byte k//4); scales are a separate array [N, K/128] (structure-of-arrays);
code 3 is rejected by the packer; f32 -> f16 rounds to nearest even and
non-finite scales are rejected; the 4-bit group is 128 with an f16 zero point
in code units; the low-rank branch has no extra scale factor; outputs are
float32 on the GPU and float64 here.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def f16_decode_scalar(bits: int) -> float:
    """IEEE 754 binary16 bit pattern -> Python float, from the format's definition
    (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits)."""
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    exp = (bits >> 10) & 0x1F
    frac = bits & 0x3FF
    if exp == 0x1F:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -24)            # subnormal: frac * 2^-14 * 2^-10
    return sign * math.ldexp(1024 + frac, exp - 25)     # (1 + frac/2^10) * 2^(exp-15)


def bf16_decode_scalar(bits: int) -> float:
    """bfloat16 bit pattern -> Python float (1 sign, 8 exponent bits with bias
    127, 7 fraction bits)."""
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -133)           # frac * 2^-126 * 2^-7
    return sign * math.ldexp(128 + frac, exp - 134)


def f16_to_f64(bits) -> np.ndarray:
    """Vectorised f16 decode: u16 bit patterns -> float64 values."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """Vectorised bf16 decode: a bf16 pattern is the top half of a float32."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Q2_0 pack (load-time conversion)
# ---------------------------------------------------------------------------

class PackError(ValueError):
    """Raised by pack_q2.  kind is 'code' or 'scale'; index is the flat
    row-major index of the first offending element of codes [N, K] or of
    scales [N, K/128].  Codes are checked before scales."""

    def __init__(self, kind: str, index: int):
        super().__init__(f"q2 pack: bad {kind} at flat index {index}")
        self.kind = kind
        self.index = index


def pack_q2(codes: np.ndarray, scales: np.ndarray):
    """codes u8 [N, K] in {0,1,2}, scales float32 [N, K/128]
    -> (packed u8 [N, K/4], scale bits u16 [N, K/128]).

    Byte j of a row holds codes 4j..4j+3, code 4j+i in bits 2i and 2i+1
    (least significant pair first).  Each scale is cast to f16 (nearest even)
    and must come back unchanged when cast back to float32; NaN and inf are
    refused.
    """
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    n, k = codes.shape
    if k % GROUP or scales.shape != (n, k // GROUP):
        raise ValueError("q2 pack: K must be a multiple of 128 and scales [N, K/128]")
    bad = np.flatnonzero(codes > 2)
    if bad.size:
        raise PackError("code", int(bad[0]))
    half = scales.astype(np.float16)
    back = half.astype(np.float32)
    ok = np.isfinite(scales) & (back == scales)
    bad = np.flatnonzero(~ok)
    if bad.size:
        raise PackError("scale", int(bad[0]))
    return pack_codes_q2(codes), half.view(np.uint16)


def pack_codes_q2(codes: np.ndarray) -> np.ndarray:
    """codes [N, K] in {0,1,2} (K a multiple of 4) -> bytes [N, K/4], byte j
    = c[4j] | c[4j+1] << 2 | c[4j+2] << 4 | c[4j+3] << 6."""
    n, k = codes.shape
    c = np.asarray(codes).reshape(n, k // 4, 4).astype(np.uint32)
    packed = c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)
    return packed.astype(np.uint8)


# ---------------------------------------------------------------------------
# Q2_0 unpack and linear
# ---------------------------------------------------------------------------

def unpack_q2_scalar(packed, scale_bits, n: int, k: int):
    """Literal per-element decode (tiny inputs only): list of rows of floats.
    q = (byte[k // 4] >> 2 (k % 4)) & 3 ;  w = (q - 1) * d[k // 128]."""
    w = []
    for row in range(n):
        out = []
        for col in range(k):
            byte = int(packed[row][col // 4])
            q = (byte >> (2 * (col % 4))) & 3
            d = f16_decode_scalar(int(scale_bits[row][col // GROUP]))
            out.append((q - 1) * d)
        w.append(out)
    return w


def codes_q2(packed: np.ndarray) -> np.ndarray:
    """u8 [N, K/4] -> codes u8 [N, K]: column k takes bits 2(k%4).. of byte k//4."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    n, kb = p.shape
    col = np.arange(kb * 4)
    return ((p[:, col // 4] >> (2 * (col % 4)).astype(np.uint8)) & 3).astype(np.uint8)


def unpack_q2(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Vectorised decode to float64 [N, K]: w[n, k] = (q[n, k] - 1) * d[n, k // 128]."""
    q = codes_q2(packed).astype(np.float64)
    d = f16_to_f64(scale_bits)
    col = np.arange(q.shape[1])
    w = (q - 1.0) * d[:, col // GROUP]
    return w + 0.0          # q == 1 with d < 0 gives -0; values compare equal either way


def q2_linear(x_bits: np.ndarray, packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """y [M, N] = X W^T in float64, X from bf16 bits [M, K]."""
    x = bf16_to_f64(x_bits)
    return x @ unpack_q2(packed, scale_bits).T


def q2_linear_cols(x_bits, packed, scale_bits, cols) -> np.ndarray:
    """The columns `cols` of q2_linear, decoding only those weight rows."""
    cols = np.asarray(cols)
    return bf16_to_f64(x_bits) @ unpack_q2(packed[cols], scale_bits[cols]).T


# ---------------------------------------------------------------------------
# Weight slices and the input-axis split
# ---------------------------------------------------------------------------
# "We're Teaching Your Browser to Paint", section "The GPU driver, and the bug
# that looked like broken math": a fused weight is cut once at load time into
# its logical row ranges, and the fused output projection, whose input is two
# activations side by side, is cut along its input axis into two products that
# are summed -- the same mathematics as the whole product.

def slice_q2(packed: np.ndarray, scale_bits: np.ndarray, n0: int, n1: int, k0: int, k1: int):
    """The Q2_0 form of the sub-matrix W[n0:n1, k0:k1] (k0, k1 multiples of
    128): its codes packed four per byte from column k0 on, and the scales of
    its whole blocks, unchanged."""
    if k0 % GROUP or k1 % GROUP:
        raise ValueError("slice_q2: input range must fall on 128-weight blocks")
    codes = codes_q2(packed)[n0:n1, k0:k1]
    return pack_codes_q2(codes), np.ascontiguousarray(scale_bits[n0:n1, k0 // GROUP:k1 // GROUP])


def q2_linear_sum(parts, y0=None) -> np.ndarray:
    """y0 (when given) plus the sum over parts of each part's linear.  A part
    is (x_bits, packed, scale_bits) or (x_bits, packed, scale_bits, a_bits,
    b_bits), as for q2_linear / q2_linear_lowrank."""
    y = None if y0 is None else np.asarray(y0, dtype=np.float64).copy()
    for part in parts:
        term = q2_linear(*part) if len(part) == 3 else q2_linear_lowrank(*part)
        y = term if y is None else y + term
    return y


# ---------------------------------------------------------------------------
# Import of a transposed, group-quantised ternary weight (gemlite-int2 style)
# ---------------------------------------------------------------------------
# "We're Teaching Your Browser to Paint", section "The lucky break that wasn't
# luck": the source stores codes {0,1,2} four per byte, least significant pair
# first, along the input axis; it dequantises with a per-group scale and zero
# point, and every zero equals minus its scale, so each weight is (q - 1) x
# scale -- the Q2_0 formula.  Conversion is a transpose and a regroup with no
# numeric change; the one rounding, the f32 -> f16 scale cast, must be exact or
# the conversion stops.  Readings (the pages give no more of the layout): the
# source is input-major -- bytes [K/4, N], byte j of column n holding codes
# 4j..4j+3 of weight row n -- with f32 scales and zeros [K/G, N]; the zero is
# a bias in weight units, w = q x scale + zero (with zero == -scale this is
# (q - 1) x scale); the group length G divides 128 or is a multiple of it,
# and a 128-weight block whose groups disagree has no Q2_0 form.

class ImportError_(ValueError):
    """Raised by import_gemlite.  kind is 'code', 'zero' or 'scale'; index is
    the flat row-major index of the first offending code in the weight [N, K]
    ('code'), or of the first offending group in the source's [K/G, N] arrays."""

    def __init__(self, kind: str, index: int):
        super().__init__(f"import: bad {kind} at flat index {index}")
        self.kind = kind
        self.index = index


def gemlite_dequant(codes_t: np.ndarray, scales_t: np.ndarray, zeros_t: np.ndarray, group: int) -> np.ndarray:
    """The source's own dequantisation, w[n, k] = q[n, k] x s[k // G, n] + z[k // G, n],
    in float64 [N, K] (exact: q is 0, 1 or 2 and s, z are f32 values)."""
    ct = np.asarray(codes_t, dtype=np.uint8)
    kq, n = ct.shape
    k = np.arange(kq * 4)
    q = ((ct[k // 4, :] >> (2 * (k % 4))[:, None].astype(np.uint8)) & 3).T.astype(np.float64)   # [N, K]
    s = np.asarray(scales_t, dtype=np.float32).astype(np.float64)[k // group, :].T
    z = np.asarray(zeros_t, dtype=np.float32).astype(np.float64)[k // group, :].T
    return q * s + z


def import_gemlite(codes_t: np.ndarray, scales_t: np.ndarray, zeros_t: np.ndarray, group: int):
    """Source (bytes [K/4, N], scales / zeros f32 [K/G, N]) -> Q2_0 (packed u8
    [N, K/4], scale bits u16 [N, K/128]).  Checks, in this order, each
    reporting its first flat index: codes <= 2; zero == -scale; the scale is a
    finite exact f16 value; within a 128-weight block every group has the same
    scale."""
    ct = np.ascontiguousarray(codes_t, dtype=np.uint8)
    st = np.ascontiguousarray(scales_t, dtype=np.float32)
    zt = np.ascontiguousarray(zeros_t, dtype=np.float32)
    kq, n = ct.shape
    k = 4 * kq
    if k % GROUP or group <= 0 or group % 4 or (GROUP % group and group % GROUP) or k % group:
        raise ValueError("import: K must be a multiple of 128 and of G; G must divide 128 or be a multiple of it")
    if st.shape != (k // group, n) or zt.shape != st.shape:
        raise ValueError("import: scales and zeros must be [K/G, N]")
    col = np.arange(k)
    codes = ((ct[col // 4, :] >> (2 * (col % 4))[:, None].astype(np.uint8)) & 3).T      # [N, K]
    bad = np.flatnonzero(codes > 2)
    if bad.size:
        raise ImportError_("code", int(bad[0]))
    bad = np.flatnonzero(~(zt == -st))
    if bad.size:
        raise ImportError_("zero", int(bad[0]))
    half = st.astype(np.float16)
    bad = np.flatnonzero(~(np.isfinite(st) & (half.astype(np.float32) == st)))
    if bad.size:
        raise ImportError_("scale", int(bad[0]))
    nb = k // GROUP
    if group < GROUP:                          # every group of a block must carry the block's scale
        per = GROUP // group
        first = st.reshape(nb, per, n)[:, :1, :]
        same = (st.reshape(nb, per, n) == first).reshape(k // group, n)
        bad = np.flatnonzero(~same)
        if bad.size:
            raise ImportError_("scale", int(bad[0]))
        block_s = st[::per, :]                  # [K/128, N]
    else:
        block_s = st[np.arange(nb) * GROUP // group, :]
    return pack_codes_q2(codes), np.ascontiguousarray(block_s.T.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------------------
# 8-bit activations
# ---------------------------------------------------------------------------
# "We're Teaching Your Browser to Paint", section "The GPU driver, and the bug
# that looked like broken math": on the GPU path the activations run through
# 8-bit quantization, which sets a few-percent error floor.  The page gives no
# more.  Readings: per-row (per-token) symmetric absmax scaling, s = amax / 127
# in float32; each code is x / s in float32, rounded to nearest even and
# clamped to [-127, 127]; a row of zeros has s = 0 and all codes 0; the
# product is y[m, n] = s[m] * sum_k xq[m, k] * w[n, k].  The codes are decided
# in float32 with IEEE division (NumPy's float32 arithmetic), as the kernel
# does.

def quantize_rows_a8(x_bits: np.ndarray):
    """bf16 bits [M, K] -> (codes int32 [M, K] in [-127, 127], scales float32 [M])."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((x / safe[:, None]).astype(np.float32))
    q = np.clip(q, -127, 127).astype(np.int32)
    q[s == 0, :] = 0
    return q, s


def q2_linear_a8(x_bits: np.ndarray, packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """y [M, N] = s[m] * (xq W^T) in float64, xq, s from quantize_rows_a8."""
    q, s = quantize_rows_a8(x_bits)
    return s.astype(np.float64)[:, None] * (q.astype(np.float64) @ unpack_q2(packed, scale_bits).T)


# ---------------------------------------------------------------------------
# Low-rank side branch  y = W x + B (A x)
# ---------------------------------------------------------------------------

def lowrank_t(x_bits: np.ndarray, a_bits: np.ndarray) -> np.ndarray:
    """t [M, r] = X A^T with A f16 [r, K]."""
    return bf16_to_f64(x_bits) @ f16_to_f64(a_bits).T


def q2_linear_lowrank(x_bits, packed, scale_bits, a_bits, b_bits) -> np.ndarray:
    """y = X W^T + (X A^T) B^T, A f16 [r, K], B f16 [N, r]; r may be 0."""
    y = q2_linear(x_bits, packed, scale_bits)
    a = np.asarray(a_bits)
    if a.size == 0:
        return y
    return y + lowrank_t(x_bits, a) @ f16_to_f64(b_bits).T


# ---------------------------------------------------------------------------
# 4-bit nibble variant
# ---------------------------------------------------------------------------

def codes_q4(packed4: np.ndarray) -> np.ndarray:
    """u8 [N, K/2] -> codes [N, K]: column k is (byte[k // 2] >> 4 (k & 1)) & 15,
    i.e. the low nibble holds the even column."""
    p = np.ascontiguousarray(packed4, dtype=np.uint8)
    col = np.arange(p.shape[1] * 2)
    return ((p[:, col // 2] >> (4 * (col & 1)).astype(np.uint8)) & 15).astype(np.uint8)


def unpack_q4(packed4, scale_bits, zero_bits) -> np.ndarray:
    """w[n, k] = (q[n, k] - z[n, k // 128]) * s[n, k // 128] in float64 (exact)."""
    q = codes_q4(packed4).astype(np.float64)
    col = np.arange(q.shape[1])
    s = f16_to_f64(scale_bits)[:, col // GROUP]
    z = f16_to_f64(zero_bits)[:, col // GROUP]
    return (q - z) * s


def q4_linear(x_bits, packed4, scale_bits, zero_bits) -> np.ndarray:
    return bf16_to_f64(x_bits) @ unpack_q4(packed4, scale_bits, zero_bits).T


def q4_linear_cols(x_bits, packed4, scale_bits, zero_bits, cols) -> np.ndarray:
    cols = np.asarray(cols)
    return bf16_to_f64(x_bits) @ unpack_q4(packed4[cols], scale_bits[cols], zero_bits[cols]).T


# ---------------------------------------------------------------------------
# Acceptance
# ---------------------------------------------------------------------------

REL_L2_TOL = 1e-4       # over the whole output
ROW_MAX_TOL = 1e-3      # per output row, relative to the oracle row's RMS


def acceptance(y, y_ref) -> dict:
    """Compare an output against the oracle.

    rel_l2 = ||y - y_ref||_2 / ||y_ref||_2 over the whole tensor;
    row_ratio = max over rows m of max_n |y - y_ref| / rms_n(y_ref[m, :]).
    A row of y_ref that is exactly zero must be matched exactly.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape {y.shape} != {y_ref.shape}")
    if y_ref.size == 0:
        return dict(rel_l2=0.0, row_ratio=0.0, ok=True)
    err = y - y_ref
    if not np.all(np.isfinite(y)):
        return dict(rel_l2=math.inf, row_ratio=math.inf, ok=False)
    ref_norm = float(np.linalg.norm(y_ref))
    rel_l2 = float(np.linalg.norm(err)) / ref_norm if ref_norm > 0 else (0.0 if not err.any() else math.inf)
    y2 = y_ref.reshape(y_ref.shape[0], -1) if y_ref.ndim > 1 else y_ref.reshape(1, -1)
    e2 = np.abs(err).reshape(y2.shape)
    rms = np.sqrt(np.mean(y2 * y2, axis=1))
    emax = e2.max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(rms > 0, emax / np.where(rms > 0, rms, 1.0), np.where(emax > 0, math.inf, 0.0))
    row_ratio = float(ratio.max())
    return dict(rel_l2=rel_l2, row_ratio=row_ratio,
                ok=bool(rel_l2 <= REL_L2_TOL and row_ratio <= ROW_MAX_TOL))
