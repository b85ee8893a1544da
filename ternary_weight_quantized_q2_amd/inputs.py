"""Seeded synthetic inputs for the Q2_0 ternary linear and its variants.

This module is the only code shared by the CPU oracle's callers and the HIP
path's callers.  It draws random numbers and stores them in the storage types
the library consumes (bf16 / f16 bit patterns, u8 codes, u8 nibble bytes); it
holds none of the method's arithmetic: no packing of 2-bit codes, no
dequantisation, no matrix products.  It imports NumPy only.

Workload recipe (stated for the synthetic stand-ins of a ~4B MMDiT denoise step
and a 4-bit text-encoder linear):

* every tensor draws from its own stream ``np.random.default_rng([0, config, tensor])``;
* Q2_0 codes are i.i.d. over {0, 1, 2} with probabilities {0.3, 0.4, 0.3};
* Q2_0 block scales are |N(0, 1)| * 0.02, rounded to the nearest f16 value and
  handed over as float32 (so the pack step's exact-roundtrip check passes);
* activations are N(0, 1) float32 rounded to bf16 (round to nearest even);
  the parity tests add four regimes that stress fp32 accumulation: N(8, 1),
  one channel at 2^12, and rows scaled by 2^100 or 2^116;
* low-rank factors A [r, K] and B [N, r] are N(0, std 0.01) rounded to f16;
* 4-bit weights are uniform random bytes, i.e. two independent codes uniform on
  0..15 per byte; their group scales are |N(0,1)| * 0.02 and zero points
  U(0, 15), both rounded to f16;
* a transposed group-quantised ternary source (for the importer) has bytes
  [K/4, N] drawn uniformly from the 81 byte values whose four 2-bit fields are
  all below 3 (so every code is i.i.d. uniform on {0, 1, 2}, whatever order the
  fields are read in), f32 group scales [K/G, N] that are f16-exact values of
  |N(0,1)| * 0.02 and equal across the groups of a 128-weight block, and zero
  points equal to minus the scales.
"""
from __future__ import annotations

import numpy as np

GROUP = 128  # weights per Q2_0 block / per 4-bit group

# tensor ids inside a config's seed tuple
T_CODES, T_SCALES, T_X, T_A, T_B, T_Q4, T_Q4S, T_Q4Z, T_SRC, T_SRCS = range(10)


def stream(config_id: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    """Independent counter-seeded stream for one tensor of one config."""
    return np.random.default_rng([seed, config_id, tensor_id])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return u16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (NumPy's nearest-even cast); u16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def q2_codes(config_id: int, n: int, k: int, p=(0.3, 0.4, 0.3)) -> np.ndarray:
    """u8 [n, k] codes in {0, 1, 2}."""
    g = stream(config_id, T_CODES)
    return g.choice(3, size=(n, k), p=list(p)).astype(np.uint8)


_DIGIT_TO_CODE = np.array([0, 0, 0, 1, 1, 1, 1, 2, 2, 2], dtype=np.uint8)


def q2_codes_fast(config_id: int, n: int, k: int) -> np.ndarray:
    """u8 [n, k] codes in {0, 1, 2} with p = (0.3, 0.4, 0.3), drawn as a uniform
    decimal digit mapped 0-2 / 3-6 / 7-9 (an order of magnitude faster than
    q2_codes, for the 100-linear layer lists)."""
    g = stream(config_id, T_CODES)
    return _DIGIT_TO_CODE[g.integers(0, 10, size=(n, k), dtype=np.uint8)]


def q2_scales(config_id: int, n: int, k: int) -> np.ndarray:
    """float32 [n, k/128] block scales whose values are exactly representable in f16."""
    g = stream(config_id, T_SCALES)
    s = np.abs(g.standard_normal((n, k // GROUP), dtype=np.float32)) * np.float32(0.02)
    return s.astype(np.float16).astype(np.float32)


def activations_bf16(config_id: int, m: int, k: int) -> np.ndarray:
    """u16 [m, k] bf16 bit patterns of N(0, 1) float32 samples."""
    g = stream(config_id, T_X)
    return f32_to_bf16_bits(g.standard_normal((m, k), dtype=np.float32))


ACT_REGIMES = ("mean8", "outlier", "huge", "near_limit")


def activations_regime_bf16(config_id: int, m: int, k: int, regime: str) -> np.ndarray:
    """u16 [m, k] bf16 bit patterns of activations that stress the fp32 sums:
    "mean8" N(8, 1) (a large common offset in every row); "outlier" N(0, 1)
    with channel k // 3 set to 2^12 in every row; "huge" N(0, 1) * 2^100;
    "near_limit" N(0, 1) * 2^116 (about 2^119 at the largest, block sums
    of |x| near 2^123)."""
    x = stream(config_id, T_X).standard_normal((m, k), dtype=np.float32)
    if regime == "mean8":
        x = x + np.float32(8.0)
    elif regime == "outlier":
        x[:, k // 3] = np.float32(4096.0)
    elif regime == "huge":
        x = x * np.float32(2.0 ** 100)
    elif regime == "near_limit":
        x = x * np.float32(2.0 ** 116)
    else:
        raise ValueError(f"unknown activation regime {regime}")
    return f32_to_bf16_bits(x)


def lowrank_factors(config_id: int, r: int, k: int, n: int, std: float = 0.01):
    """(A u16 [r, k], B u16 [n, r]) f16 bit patterns of N(0, std) samples."""
    a = stream(config_id, T_A).standard_normal((r, k), dtype=np.float32) * np.float32(std)
    b = stream(config_id, T_B).standard_normal((n, r), dtype=np.float32) * np.float32(std)
    return f32_to_f16_bits(a), f32_to_f16_bits(b)


def q4_weights(config_id: int, n: int, k: int):
    """(bytes u8 [n, k/2], scale u16 [n, k/128], zero u16 [n, k/128]).

    Bytes are uniform on 0..255, which makes both 4-bit codes of a byte
    independent and uniform on 0..15 whatever order they are read in.
    """
    g = stream(config_id, T_Q4)
    p4 = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    s = np.abs(stream(config_id, T_Q4S).standard_normal((n, k // GROUP), dtype=np.float32))
    z = stream(config_id, T_Q4Z).uniform(0.0, 15.0, size=(n, k // GROUP)).astype(np.float32)
    return p4, f32_to_f16_bits(s * np.float32(0.02)), f32_to_f16_bits(z)


# The five workload families, with their shapes.
CONFIG_TINY = dict(id=1, M=4, K=256, N=64)
GEMV_SHAPES = [(3072, 3072), (3072, 9216), (3072, 12288), (12288, 3072)]   # (K, N), M = 1
GEMM_M = 1536                                                              # 1024 image + 512 text tokens
GEMM_SHAPES = [(3072, 3072), (3072, 9216), (3072, 12288), (12288, 3072)]   # (K, N)
LOWRANK = dict(M=1536, K=3072, N=9216, ranks=(4, 32, 64), linears=100, steps=4)
# The quarter-size first step of the two-step schedule: 256 image patches and
# 128 text rows; joint blocks run the two streams through their own weights
# (M = 256 and M = 128), single blocks run them together (M = 384).
QUARTER_M = (384, 256, 128)
Q4_M = 128
Q4_SHAPES = [(2560, 9728), (9728, 2560), (2560, 2560)]                     # (K, N)


# Byte values whose four 2-bit fields are all in {0, 1, 2}.
_TERNARY_BYTES = np.array([b for b in range(256) if all((b >> (2 * f)) & 3 != 3 for f in range(4))], np.uint8)


def gemlite_source(config_id: int, n: int, k: int, group: int):
    """(bytes u8 [k/4, n], scales f32 [k/group, n], zeros f32 [k/group, n]): a
    valid transposed group-quantised ternary weight for the importer."""
    b = _TERNARY_BYTES[stream(config_id, T_SRC).integers(0, len(_TERNARY_BYTES), size=(k // 4, n))]
    blocks = np.abs(stream(config_id, T_SRCS).standard_normal((k // GROUP, n), dtype=np.float32)) * np.float32(0.02)
    blocks = blocks.astype(np.float16).astype(np.float32)
    if group < GROUP:
        scales = np.repeat(blocks, GROUP // group, axis=0)
    else:
        scales = blocks[::group // GROUP]
    scales = np.ascontiguousarray(scales)
    return np.ascontiguousarray(b), scales, np.ascontiguousarray(-scales)
