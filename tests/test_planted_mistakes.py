"""Each pin must catch a plausible mistake.  The mistakes are planted in copies
of the oracle's functions, on the CPU; the pins are the check_* functions of
test_oracle_pins run against those copies."""
import numpy as np
import pytest

import oracle.q2_oracle as O
from tests import test_oracle_pins as P


def unpack_msb_first(packed, sc):
    p = np.asarray(packed)
    col = np.arange(p.shape[1] * 4)
    q = (p[:, col // 4] >> (6 - 2 * (col % 4)).astype(np.uint8)) & 3
    return (q - 1.0) * O.f16_to_f64(sc)[:, col // 128]


def unpack_no_offset(packed, sc):            # (q) * d instead of (q - 1) * d
    return O.unpack_q2(packed, sc) + O.f16_to_f64(sc)[:, np.arange(np.asarray(packed).shape[1] * 4) // 128]


def unpack_block64(packed, sc):              # scale index with the wrong block length
    q = O.codes_q2(packed).astype(np.float64)
    col = np.arange(q.shape[1])
    d = O.f16_to_f64(sc)
    return (q - 1.0) * d[:, np.minimum(col // 64, d.shape[1] - 1)]


def linear_with(unpack):
    return lambda xb, p, s: O.bf16_to_f64(xb) @ unpack(p, s).T


def pack_msb_first(codes, scales):
    p, s = O.pack_q2(codes, scales)
    c = np.asarray(codes).reshape(codes.shape[0], -1, 4).astype(np.uint32)
    return (c[..., 3] | c[..., 2] << 2 | c[..., 1] << 4 | c[..., 0] << 6).astype(np.uint8), s


def lowrank_b_transposed(xb, p, s, a, b):
    y = O.q2_linear(xb, p, s)
    if np.asarray(a).size == 0:
        return y
    return y + O.lowrank_t(xb, a) @ O.f16_to_f64(b)


def lowrank_dropped_branch(xb, p, s, a, b):
    return O.q2_linear(xb, p, s)


def q4_swapped_nibbles(xb, p4, s, z):
    p = np.asarray(p4)
    swapped = ((p >> 4) | (p << 4)).astype(np.uint8)
    return O.q4_linear(xb, swapped, s, z)


def q4_zero_sign(xb, p4, s, z):              # (q + z) * s
    q = O.codes_q4(p4).astype(np.float64)
    col = np.arange(q.shape[1])
    w = (q + O.f16_to_f64(z)[:, col // 128]) * O.f16_to_f64(s)[:, col // 128]
    return O.bf16_to_f64(xb) @ w.T


def slice_scales_at_input_column(packed, sc, n0, n1, k0, k1):     # scale index k0 instead of k0 / 128
    sp, _ = O.slice_q2(packed, sc, n0, n1, k0, k1)
    nb = (k1 - k0) // 128
    cols = np.minimum(np.arange(k0, k0 + nb), np.asarray(sc).shape[1] - 1)
    return sp, np.ascontiguousarray(np.asarray(sc)[n0:n1][:, cols])


def slice_codes_at_byte_k0(packed, sc, n0, n1, k0, k1):           # byte offset k0 instead of k0 / 4
    _, ss = O.slice_q2(packed, sc, n0, n1, k0, k1)
    p = np.asarray(packed)
    start = min(k0, p.shape[1] - (k1 - k0) // 4)
    return np.ascontiguousarray(p[n0:n1, start:start + (k1 - k0) // 4]), ss


def import_no_transpose(ct, st, zt, group):          # source bytes read as if already [N, K/4]
    p, s = O.import_gemlite(ct, st, zt, group)
    flat = np.ascontiguousarray(ct).reshape(-1)[:p.size]
    return flat.reshape(p.shape).copy(), s


def import_zero_plus_scale(ct, st, zt, group):      # accepts zero == +scale as well
    zt = np.where(np.asarray(zt) == np.asarray(st), -np.asarray(st), zt)
    return O.import_gemlite(ct, st, zt, group)


def import_regroup_unchecked(ct, st, zt, group):    # takes each block's first group, never compares
    if group < 128:
        per = 128 // group
        st = np.repeat(np.asarray(st)[::per], per, axis=0)
        zt = -st
    return O.import_gemlite(ct, st, zt, group)


def a8_truncating(xb):                              # codes truncated instead of rounded
    x = (np.asarray(xb, np.uint16).astype(np.uint32) << 16).view(np.float32)
    _, s = O.quantize_rows_a8(xb)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.clip(np.trunc(x / safe[:, None]), -127, 127).astype(np.int32)
    q[s == 0] = 0
    return q, s


def a8_per_tensor(xb):                              # one scale for the whole matrix
    x = (np.asarray(xb, np.uint16).astype(np.uint32) << 16).view(np.float32)
    amax = np.float32(np.abs(x).max())
    s = np.full(x.shape[0], amax / np.float32(127), np.float32)
    q = np.clip(np.rint(x / s[:, None]), -127, 127).astype(np.int32)
    return q, s


def a8_unsigned_range(xb):                          # scale for 255 levels
    q, s = O.quantize_rows_a8(xb)
    x = (np.asarray(xb, np.uint16).astype(np.uint32) << 16).view(np.float32)
    s2 = (np.max(np.abs(x), axis=1) / np.float32(255)).astype(np.float32)
    safe = np.where(s2 > 0, s2, np.float32(1)).astype(np.float32)
    return np.clip(np.rint(x / safe[:, None]), -255, 255).astype(np.int32), s2


def a8_scale_dropped(xb, p, s):                     # the row scale never applied
    q, _ = O.quantize_rows_a8(xb)
    return q.astype(np.float64) @ O.unpack_q2(p, s).T


def q4_cols_shifted(xb, p4, s, z, cols):           # the neighbouring weight rows
    c = (np.asarray(cols) + 1) % np.asarray(p4).shape[0]
    return O.q4_linear(xb, p4[c], s[c], z[c])


def q4_cols_no_zero(xb, p4, s, z, cols):           # q * s: the zero point dropped
    c = np.asarray(cols)
    return O.q4_linear(xb, p4[c], s[c], np.zeros_like(np.asarray(z)[c]))


def import_codes_reversed(ct, st, zt, g):          # codes of each byte taken MSB-first
    p, s = O.import_gemlite(ct, st, zt, g)
    c = O.codes_q2(p).reshape(p.shape[0], -1, 4)[..., ::-1].reshape(p.shape[0], -1)
    return O.pack_codes_q2(c), s


MUTANTS = {
    "q4 columns shifted": lambda: P.check_q4_cols(q4_cols_shifted),
    "q4 columns without zero point": lambda: P.check_q4_cols(q4_cols_no_zero),
    "import codes reversed in each byte": lambda: P.check_import(import_codes_reversed),
    "a8 truncating": lambda: P.check_a8(a8_truncating, O.q2_linear_a8),
    "a8 per-tensor scale": lambda: P.check_a8(a8_per_tensor, O.q2_linear_a8),
    "a8 255 levels": lambda: P.check_a8(a8_unsigned_range, O.q2_linear_a8),
    "a8 row scale dropped": lambda: P.check_a8(O.quantize_rows_a8, a8_scale_dropped),
    "import without the transpose": lambda: P.check_import(import_no_transpose),
    "import accepts zero == +scale": lambda: P.check_import(import_zero_plus_scale),
    "import regroups without comparing": lambda: P.check_import(import_regroup_unchecked),
    "slice scales at the input column": lambda: P.check_slice(slice_scales_at_input_column),
    "slice codes at byte k0": lambda: P.check_slice(slice_codes_at_byte_k0),
    "split sum drops y0": lambda: P.check_split_sum(lambda parts, y0=None: O.q2_linear_sum(parts)),
    "split sum adds y0 twice": lambda: P.check_split_sum(
        lambda parts, y0=None: O.q2_linear_sum(parts, y0) + (0 if y0 is None else y0)),
    "split sum drops the second part": lambda: P.check_split_sum(lambda parts, y0=None: O.q2_linear_sum(parts[:1], y0)),
    "unpack MSB-first": lambda: P.check_q2_bit_order(O.pack_q2, unpack_msb_first, linear_with(unpack_msb_first)),
    "pack MSB-first": lambda: P.check_q2_bit_order(pack_msb_first, O.unpack_q2, O.q2_linear),
    "zero point 0": lambda: P.check_q2_closed_forms(linear_with(unpack_no_offset)),
    "block length 64": lambda: P.check_q2_closed_forms(linear_with(unpack_block64)),
    "block length 64 (brute force)": lambda: P.check_q2_exact_bruteforce(linear_with(unpack_block64)),
    "input axis reversed": lambda: P.check_q2_exact_bruteforce(lambda xb, p, s: O.bf16_to_f64(xb) @ O.unpack_q2(p, s)[:, ::-1].T),
    "rows and columns swapped": lambda: P.check_q2_exact_bruteforce(lambda xb, p, s: (O.bf16_to_f64(xb) @ O.unpack_q2(p, s).T)[::-1]),
    "low-rank B transposed": lambda: P.check_lowrank(lowrank_b_transposed),
    "low-rank branch dropped": lambda: P.check_lowrank(lowrank_dropped_branch),
    "q4 nibbles swapped": lambda: P.check_q4(q4_swapped_nibbles),
    "q4 zero sign": lambda: P.check_q4(q4_zero_sign),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pin_catches(name):
    with pytest.raises(Exception):
        MUTANTS[name]()


def test_unmutated_checks_pass():
    P.check_q2_bit_order(O.pack_q2, O.unpack_q2, O.q2_linear)
    P.check_q2_closed_forms(O.q2_linear)
    P.check_lowrank(O.q2_linear_lowrank)
    P.check_q4(O.q4_linear)
    P.check_q4_cols(O.q4_linear_cols)
    P.check_slice(O.slice_q2)
    P.check_split_sum(O.q2_linear_sum)
    P.check_import(O.import_gemlite)
    P.check_a8(O.quantize_rows_a8, O.q2_linear_a8)
