"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/q2.h declares, and rejects bad arguments before any HIP
call.  No compute entry point is driven past its argument checks here."""
import ctypes
import os
import re

import pytest

import ternary_weight_quantized_q2_amd as q2
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "q2.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(q[24]_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return q2.load()


def test_header_declares_the_expected_entry_points():
    assert header_functions() == sorted(q2.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_strerror_and_workspace_size(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert lib.q2_strerror(st)
    assert b"unknown" in lib.q2_strerror(-99)
    assert lib.q2_lowrank_workspace_bytes(0, 32) == 0
    assert lib.q2_lowrank_workspace_bytes(1536, 0) == 0
    assert lib.q2_lowrank_workspace_bytes(-1, 5) == 0
    assert lib.q2_lowrank_workspace_bytes(1, 4) == 256
    assert lib.q2_lowrank_workspace_bytes(1536, 64) == 1536 * 64 * 4
    assert lib.q2_lowrank_workspace_bytes(3, 5) == 256
    assert lib.q2_lowrank_workspace_bytes(100, 5) == 100 * 8 * 4 // 256 * 256 + 256     # r padded to 8
    assert lib.q2_lowrank_workspace_bytes(1000, 33) == 1000 * 40 * 4


def test_noalloc_argument_errors(lib):
    # checked before any HIP call: sizes beyond the fixed scratch, then the usual argument errors
    st = lib.q2_linear_lowrank_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 65536, 128, 128, None)
    assert st == q2.Q2_ERR_WORKSPACE
    assert lib.q2_linear_lowrank_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 4, 128, 128, None) == q2.Q2_ERR_ARG
    assert lib.q2_linear_lowrank_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 128, 100, None) == q2.Q2_ERR_SHAPE
    assert lib.q2_linear_lowrank_noalloc(None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 128, 128, None) == q2.Q2_ERR_ARG
    assert lib.q2_linear_lowrank_noalloc(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 128, 128, None) == q2.Q2_ERR_ALIGN
    assert lib.q2_linear_lowrank_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, 128, 128, None) == q2.Q2_OK


def test_set_dispatch_arguments(lib):
    # no HIP call is involved: names are checked and stored on the host
    assert lib.q2_set_dispatch(b"gemv", b"kg6x3x2", 2) == q2.Q2_OK
    assert lib.q2_set_dispatch(b"bogus", None, 0) == q2.Q2_ERR_ARG
    assert lib.q2_set_dispatch(None, b"no-such-tile", 0) == q2.Q2_ERR_ARG
    assert lib.q2_set_dispatch(None, None, 3) == q2.Q2_ERR_ARG
    assert lib.q2_set_dispatch(b"auto", b"", 0) == q2.Q2_OK
    assert lib.q2_set_dispatch(None, None, 0) == q2.Q2_OK


FAKE = 1 << 20          # 16-byte aligned fake device address (never dereferenced)


def test_linear_argument_errors(lib):
    L = lib.q2_linear
    assert L(FAKE, FAKE, FAKE, FAKE, -1, 8, 128, None) == q2.Q2_ERR_ARG
    assert L(FAKE, FAKE, FAKE, FAKE, 4, 8, 100, None) == q2.Q2_ERR_SHAPE
    assert L(None, FAKE, FAKE, FAKE, 4, 8, 128, None) == q2.Q2_ERR_ARG
    assert L(FAKE, None, FAKE, FAKE, 4, 8, 128, None) == q2.Q2_ERR_ARG
    assert L(FAKE, FAKE, FAKE, None, 4, 8, 128, None) == q2.Q2_ERR_ARG
    assert L(FAKE + 8, FAKE, FAKE, FAKE, 4, 8, 128, None) == q2.Q2_ERR_ALIGN
    assert L(FAKE, FAKE + 4, FAKE, FAKE, 4, 8, 128, None) == q2.Q2_ERR_ALIGN
    assert L(FAKE, FAKE, FAKE + 1, FAKE, 4, 8, 128, None) == q2.Q2_ERR_ALIGN
    assert L(FAKE, FAKE, FAKE, FAKE + 2, 4, 8, 128, None) == q2.Q2_ERR_ALIGN
    assert L(FAKE, FAKE, FAKE, FAKE, 4, 8, 100, None) == q2.Q2_ERR_SHAPE and b"K=100" in lib.q2_last_error()
    # empty problems are valid no-ops that touch nothing, NULL pointers allowed
    assert L(None, FAKE, FAKE, None, 0, 8, 128, None) == q2.Q2_OK
    assert L(FAKE, None, None, None, 4, 0, 128, None) == q2.Q2_OK
    assert L(None, None, None, None, 0, 0, 0, None) == q2.Q2_OK
    assert L(None, FAKE, FAKE, None, 0, 8, 128, None) == q2.Q2_OK
    assert lib.q4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 5, 64, None) == q2.Q2_ERR_SHAPE
    assert lib.q4_linear(FAKE, FAKE, FAKE, None, FAKE, 3, 5, 128, None) == q2.Q2_ERR_ARG
    assert lib.q2_dequant(FAKE, FAKE, FAKE, 4, 130, None) == q2.Q2_ERR_SHAPE
    # K beyond 2^24 is refused by every linear entry point (checked before any HIP call)
    big = (1 << 24) + 128
    assert L(FAKE, FAKE, FAKE, FAKE, 4, 8, big, None) == q2.Q2_ERR_SHAPE and b"16777216" in lib.q2_last_error()
    assert lib.q4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, big, None) == q2.Q2_ERR_SHAPE
    assert lib.q2_linear_lowrank(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 4, 8, big, FAKE, 1 << 20,
                                 None) == q2.Q2_ERR_SHAPE
    assert lib.q2_dequant(None, None, None, 0, 128, None) == q2.Q2_OK


def test_lowrank_argument_errors(lib):
    LR = lib.q2_linear_lowrank
    need = lib.q2_lowrank_workspace_bytes(16, 8)
    assert LR(FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 16, 8, 128, FAKE, need, None) == q2.Q2_ERR_ARG
    assert LR(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 128, FAKE, need - 1, None) == q2.Q2_ERR_WORKSPACE
    assert LR(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 128, FAKE + 16, need, None) == q2.Q2_ERR_ALIGN
    assert LR(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 128, None, need, None) == q2.Q2_ERR_ARG
    assert LR(FAKE, FAKE, FAKE, FAKE + 2, FAKE, 8, FAKE, 16, 8, 128, FAKE, need, None) == q2.Q2_ERR_ALIGN
    assert LR(FAKE, FAKE, FAKE, None, FAKE, 8, FAKE, 16, 8, 128, FAKE, need, None) == q2.Q2_ERR_ARG
    assert LR(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 96, FAKE, need, None) == q2.Q2_ERR_SHAPE


def test_linear_ex_argument_errors(lib):
    E = lib.q2_linear_ex
    need = lib.q2_lowrank_workspace_bytes(16, 8)
    acc = q2.Q2_ACCUMULATE
    # unknown flag bits, then the q2_linear / q2_linear_lowrank rules
    assert E(FAKE, FAKE, FAKE, None, None, 0, FAKE, 16, 8, 128, None, 0, 2, None) == q2.Q2_ERR_ARG
    assert b"flag" in lib.q2_last_error()
    assert E(FAKE, FAKE, FAKE, None, None, 0, FAKE, 16, 8, 100, None, 0, acc, None) == q2.Q2_ERR_SHAPE
    assert E(FAKE, FAKE, FAKE, None, None, 0, None, 16, 8, 128, None, 0, acc, None) == q2.Q2_ERR_ARG
    assert E(FAKE, FAKE, FAKE, None, None, 0, FAKE + 2, 16, 8, 128, None, 0, acc, None) == q2.Q2_ERR_ALIGN
    assert E(FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 16, 8, 128, FAKE, need, acc, None) == q2.Q2_ERR_ARG
    assert E(FAKE, FAKE, FAKE, None, FAKE, 8, FAKE, 16, 8, 128, FAKE, need, acc, None) == q2.Q2_ERR_ARG
    assert E(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 128, FAKE, need - 1, acc, None) == q2.Q2_ERR_WORKSPACE
    assert E(FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 16, 8, 128, FAKE + 16, need, acc, None) == q2.Q2_ERR_ALIGN
    # r == 0 ignores A, B and the workspace; empty problems and an empty sum added touch nothing
    assert E(None, FAKE, FAKE, None, None, 0, None, 0, 8, 128, None, 0, acc, None) == q2.Q2_OK
    assert E(FAKE, None, None, None, None, 0, FAKE, 16, 8, 0, None, 0, acc, None) == q2.Q2_OK


def test_slice_argument_errors(lib):
    S = lib.q2_slice
    assert S(FAKE, FAKE, 8, 512, 0, 9, 0, 128, FAKE, FAKE, None) == q2.Q2_ERR_ARG       # n1 > N
    assert S(FAKE, FAKE, 8, 512, 5, 4, 0, 128, FAKE, FAKE, None) == q2.Q2_ERR_ARG       # n1 < n0
    assert S(FAKE, FAKE, 8, 512, -1, 4, 0, 128, FAKE, FAKE, None) == q2.Q2_ERR_ARG
    assert S(FAKE, FAKE, 8, 512, 0, 4, 256, 128, FAKE, FAKE, None) == q2.Q2_ERR_ARG     # k1 < k0
    assert S(FAKE, FAKE, 8, 512, 0, 4, 0, 640, FAKE, FAKE, None) == q2.Q2_ERR_ARG       # k1 > K
    assert S(FAKE, FAKE, 8, 512, 0, 4, 64, 256, FAKE, FAKE, None) == q2.Q2_ERR_SHAPE    # not on a block boundary
    assert b"block" in lib.q2_last_error()
    assert S(FAKE, FAKE, 8, 500, 0, 4, 0, 128, FAKE, FAKE, None) == q2.Q2_ERR_SHAPE     # K itself
    assert S(FAKE, FAKE, 8, 512, 0, 4, 0, 128, FAKE + 4, FAKE, None) == q2.Q2_ERR_ALIGN
    assert S(FAKE, FAKE, 8, 512, 0, 4, 0, 128, FAKE, FAKE + 1, None) == q2.Q2_ERR_ALIGN
    assert S(FAKE, None, 8, 512, 0, 4, 0, 128, FAKE, FAKE, None) == q2.Q2_ERR_ARG
    assert S(FAKE, FAKE, 8, 512, 0, 4, 0, 128, None, FAKE, None) == q2.Q2_ERR_ARG
    # empty ranges do nothing, NULL pointers allowed
    assert S(None, None, 8, 512, 3, 3, 0, 128, None, None, None) == q2.Q2_OK
    assert S(None, None, 8, 512, 0, 8, 256, 256, None, None, None) == q2.Q2_OK


def test_a8_argument_errors(lib):
    A8 = lib.q2_linear_a8
    assert lib.q2_a8_workspace_bytes(0, 128) == 0 and lib.q2_a8_workspace_bytes(4, 0) == 0
    assert lib.q2_a8_workspace_bytes(3, 128) == 512 + 256            # int8 codes, then row scales
    assert lib.q2_a8_workspace_bytes(1536, 3072) == 1536 * 3072 + 1536 * 4
    need = lib.q2_a8_workspace_bytes(16, 256)
    assert A8(FAKE, FAKE, FAKE, FAKE, 16, 8, 100, FAKE, need, None) == q2.Q2_ERR_SHAPE
    assert A8(FAKE, FAKE, FAKE, FAKE, 16, 8, 256, FAKE, need - 1, None) == q2.Q2_ERR_WORKSPACE
    assert A8(FAKE, FAKE, FAKE, FAKE, 16, 8, 256, None, need, None) == q2.Q2_ERR_ARG
    assert A8(FAKE, FAKE, FAKE, FAKE, 16, 8, 256, FAKE + 16, need, None) == q2.Q2_ERR_ALIGN
    assert A8(FAKE + 8, FAKE, FAKE, FAKE, 16, 8, 256, FAKE, need, None) == q2.Q2_ERR_ALIGN
    assert A8(None, FAKE, FAKE, FAKE, 16, 8, 256, FAKE, need, None) == q2.Q2_ERR_ARG
    assert A8(None, FAKE, FAKE, None, 0, 8, 256, None, 0, None) == q2.Q2_OK


def test_import_argument_errors(lib):
    I_ = lib.q2_import_gemlite
    bad = ctypes.c_int64(123)
    assert I_(FAKE, FAKE, FAKE, 8, 512, 48, FAKE, FAKE, ctypes.byref(bad), None) == q2.Q2_ERR_SHAPE   # G
    assert bad.value == -1
    assert I_(FAKE, FAKE, FAKE, 8, 384, 256, FAKE, FAKE, None, None) == q2.Q2_ERR_SHAPE     # G does not divide K
    assert I_(FAKE, FAKE, FAKE, 8, 500, 64, FAKE, FAKE, None, None) == q2.Q2_ERR_SHAPE      # K
    assert I_(FAKE, FAKE, FAKE, 8, 512, 0, FAKE, FAKE, None, None) == q2.Q2_ERR_SHAPE
    assert I_(FAKE, FAKE, FAKE, -1, 512, 64, FAKE, FAKE, None, None) == q2.Q2_ERR_ARG
    assert I_(FAKE, FAKE + 2, FAKE, 8, 512, 64, FAKE, FAKE, None, None) == q2.Q2_ERR_ALIGN
    assert I_(FAKE, FAKE, FAKE, 8, 512, 64, FAKE + 4, FAKE, None, None) == q2.Q2_ERR_ALIGN
    assert I_(None, FAKE, FAKE, 8, 512, 64, FAKE, FAKE, None, None) == q2.Q2_ERR_ARG
    assert I_(None, None, None, 0, 512, 64, None, None, None, None) == q2.Q2_OK
    assert I_(None, None, None, 8, 0, 64, None, None, None, None) == q2.Q2_OK


def test_pack_argument_errors(lib):
    bad = ctypes.c_int64(123)
    P = lib.q2_pack
    assert P(FAKE, FAKE, 4, 100, FAKE, FAKE, ctypes.byref(bad), None) == q2.Q2_ERR_SHAPE
    assert bad.value == -1
    assert P(FAKE + 4, FAKE, 4, 128, FAKE, FAKE, None, None) == q2.Q2_ERR_ALIGN
    assert P(FAKE, None, 4, 128, FAKE, FAKE, None, None) == q2.Q2_ERR_ARG
    assert P(None, None, 0, 128, None, None, None, None) == q2.Q2_OK


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "ternary_weight_quantized_q2_amd")
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle)|q2_oracle|oracle[/.]", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                assert not pat.search(open(os.path.join(dirpath, f)).read()), f


def test_binding_fails_loudly_without_the_library(tmp_path):
    saved = q2._lib
    q2._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            q2.load(str(tmp_path / "missing.so"))
    finally:
        q2._lib = saved
