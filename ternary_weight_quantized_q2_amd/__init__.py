"""Python binding of libq2 (the Q2_0 ternary linear for gfx950).

Argument marshalling only: every function hands torch tensors' device
pointers, sizes and torch's current HIP stream to the C ABI declared in
include/q2.h; all arithmetic runs in the library's HIP kernels.  Output
tensors are allocated with torch when the caller does not pass them.  The
library is loaded lazily; a missing or unloadable library raises at the first
call, never falls back to anything else.

Tensor conventions: activations torch.bfloat16 [M, K]; Q2_0 codes torch.uint8
[N, K/4]; scales, low-rank factors and 4-bit scales / zeros torch.float16;
outputs torch.float32.  All tensors must be contiguous and on the current
device.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# Q2_LIB names another build of the same library (for A/B measurements).
LIB_PATH = os.environ.get("Q2_LIB") or os.path.join(_HERE, "libq2.so")

Q2_OK, Q2_ERR_ARG, Q2_ERR_SHAPE, Q2_ERR_ALIGN, Q2_ERR_CODE, Q2_ERR_SCALE, Q2_ERR_DEVICE, Q2_ERR_HIP, \
    Q2_ERR_WORKSPACE, Q2_ERR_FORMAT = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9

Q2_ACCUMULATE = 0x1      # q2_linear_ex flag: y += result

EXPORTS = ("q2_pack", "q2_import_gemlite", "q2_linear", "q2_lowrank_workspace_bytes", "q2_linear_lowrank", "q2_linear_lowrank_noalloc",
           "q2_linear_ex", "q2_slice",
           "q2_a8_workspace_bytes", "q2_linear_a8",
           "q4_linear", "q2_dequant", "q2_set_dispatch", "q2_strerror", "q2_last_error")

_lib = None


class Q2Error(RuntimeError):
    def __init__(self, status: int, message: str, bad_index: int = -1):
        super().__init__(message)
        self.status = status
        self.bad_index = bad_index


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libq2.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libq2 is not built ({path} missing): run "
                           "`python -m ternary_weight_quantized_q2_amd.build_lib`")
    lib = ctypes.CDLL(path)
    p, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "q2_pack": ([p, p, i64, i64, p, p, ctypes.POINTER(ctypes.c_int64), p], ctypes.c_int),
        "q2_import_gemlite": ([p, p, p, i64, i64, i64, p, p, ctypes.POINTER(ctypes.c_int64), p], ctypes.c_int),
        "q2_linear": ([p, p, p, p, i64, i64, i64, p], ctypes.c_int),
        "q2_lowrank_workspace_bytes": ([i64, i64], sz),
        "q2_linear_lowrank": ([p, p, p, p, p, i64, p, i64, i64, i64, p, sz, p], ctypes.c_int),
        "q2_linear_lowrank_noalloc": ([p, p, p, p, p, i64, p, i64, i64, i64, p], ctypes.c_int),
        "q2_linear_ex": ([p, p, p, p, p, i64, p, i64, i64, i64, p, sz, ctypes.c_uint32, p], ctypes.c_int),
        "q2_slice": ([p, p, i64, i64, i64, i64, i64, i64, p, p, p], ctypes.c_int),
        "q2_a8_workspace_bytes": ([i64, i64], sz),
        "q2_linear_a8": ([p, p, p, p, i64, i64, i64, p, sz, p], ctypes.c_int),
        "q4_linear": ([p, p, p, p, p, i64, i64, i64, p], ctypes.c_int),
        "q2_dequant": ([p, p, p, i64, i64, p], ctypes.c_int),
        "q2_set_dispatch": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int], ctypes.c_int),
        "q2_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "q2_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(status: int, bad_index: int = -1) -> None:
    if status != Q2_OK:
        lib = load()
        msg = f"{lib.q2_strerror(status).decode()}: {lib.q2_last_error().decode()}"
        raise Q2Error(status, msg, bad_index)


def _ptr(t) -> int | None:
    return None if t is None else (t.data_ptr() or None)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _want(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def q2_pack(codes: torch.Tensor, scales: torch.Tensor, packed=None, scales_f16=None):
    """codes u8 [N, K] in {0,1,2}, scales f32 [N, K/128] -> (packed u8 [N, K/4], scales f16 [N, K/128])."""
    lib = load()
    n, k = codes.shape
    _want(codes, torch.uint8, (n, k), "codes")
    _want(scales, torch.float32, (n, k // 128), "scales")
    dev = codes.device
    if packed is None:
        packed = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
    if scales_f16 is None:
        scales_f16 = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
    bad = ctypes.c_int64(-1)
    st = lib.q2_pack(_ptr(codes), _ptr(scales), n, k, _ptr(packed), _ptr(scales_f16), ctypes.byref(bad), _stream())
    _check(st, bad.value)
    return packed, scales_f16


def q2_import_gemlite(codes_t, scales_t, zeros_t, group: int, packed=None, scales_f16=None):
    """Transposed group-quantised ternary weight -> Q2_0: codes_t u8 [K/4, N] (input-major),
    scales_t / zeros_t f32 [K/G, N] -> (packed u8 [N, K/4], scales f16 [N, K/128])."""
    lib = load()
    kq, n = codes_t.shape
    k = kq * 4
    _want(codes_t, torch.uint8, (kq, n), "codes_t")
    g = max(int(group), 1)
    _want(scales_t, torch.float32, (k // g, n), "scales_t")
    _want(zeros_t, torch.float32, (k // g, n), "zeros_t")
    dev = codes_t.device
    if packed is None:
        packed = torch.empty((n, kq), dtype=torch.uint8, device=dev)
    if scales_f16 is None:
        scales_f16 = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
    bad = ctypes.c_int64(-1)
    st = lib.q2_import_gemlite(_ptr(codes_t), _ptr(scales_t), _ptr(zeros_t), n, k, int(group), _ptr(packed),
                               _ptr(scales_f16), ctypes.byref(bad), _stream())
    _check(st, bad.value)
    return packed, scales_f16


def q2_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, y=None) -> torch.Tensor:
    """y [M, N] f32 = x W^T for Q2_0 weights (packed u8 [N, K/4], scales f16 [N, K/128])."""
    lib = load()
    m, k = x.shape
    n = packed.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed, torch.uint8, (n, k // 4), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    _check(lib.q2_linear(_ptr(x), _ptr(packed), _ptr(scales), _ptr(y), m, n, k, _stream()))
    return y


def lowrank_workspace_bytes(m: int, r: int) -> int:
    return int(load().q2_lowrank_workspace_bytes(m, r))


def q2_linear_lowrank(x, packed, scales, A, B, y=None, workspace=None) -> torch.Tensor:
    """y = x W^T + (x A^T) B^T; A f16 [r, K], B f16 [N, r]."""
    lib = load()
    m, k = x.shape
    n = packed.shape[0]
    r = A.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed, torch.uint8, (n, k // 4), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    _want(A, torch.float16, (r, k), "A")
    _want(B, torch.float16, (n, r), "B")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    need = lowrank_workspace_bytes(m, r)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib.q2_linear_lowrank(_ptr(x), _ptr(packed), _ptr(scales), _ptr(A), _ptr(B), r, _ptr(y), m, n, k,
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    _check(st)
    return y


NOALLOC_SCRATCH_BYTES = 8388608      # Q2_NOALLOC_SCRATCH_BYTES


def q2_linear_lowrank_noalloc(x, packed, scales, A, B, y=None) -> torch.Tensor:
    """q2_linear_lowrank with the library's per-device scratch instead of a workspace (no allocation in the
    library; y is allocated here only when not given)."""
    lib = load()
    m, k = x.shape
    n = packed.shape[0]
    r = A.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed, torch.uint8, (n, k // 4), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    _want(A, torch.float16, (r, k), "A")
    _want(B, torch.float16, (n, r), "B")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    _check(lib.q2_linear_lowrank_noalloc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(A), _ptr(B), r, _ptr(y), m, n, k,
                                         _stream()))
    return y


def q2_linear_ex(x, packed, scales, y=None, A=None, B=None, accumulate=False, workspace=None) -> torch.Tensor:
    """q2_linear (A, B None) or q2_linear_lowrank with flags; accumulate=True adds the result into y,
    which must then be given."""
    lib = load()
    m, k = x.shape
    n = packed.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed, torch.uint8, (n, k // 4), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    if (A is None) != (B is None):
        raise ValueError("A and B come together")
    r = 0 if A is None else A.shape[0]
    if r:
        _want(A, torch.float16, (r, k), "A")
        _want(B, torch.float16, (n, r), "B")
    if y is None:
        if accumulate:
            raise ValueError("accumulate=True needs y")
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    ws_bytes = 0
    if r:
        need = lowrank_workspace_bytes(m, r)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.q2_linear_ex(_ptr(x), _ptr(packed), _ptr(scales), _ptr(A), _ptr(B), r, _ptr(y), m, n, k,
                          _ptr(workspace), ws_bytes, Q2_ACCUMULATE if accumulate else 0, _stream())
    _check(st)
    return y


def q2_slice(packed, scales, n0: int, n1: int, k0: int, k1: int, out=None, out_scales=None):
    """Rows [n0, n1) and inputs [k0, k1) (multiples of 128) of a packed Q2_0 weight, as a new dense
    packed weight: (packed u8 [n1-n0, (k1-k0)/4], scales f16 [n1-n0, (k1-k0)/128])."""
    lib = load()
    n, kq = packed.shape
    k = kq * 4
    _want(packed, torch.uint8, (n, kq), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    rows, ks = max(n1 - n0, 0), max(k1 - k0, 0)
    dev = packed.device
    if out is None:
        out = torch.empty((rows, ks // 4), dtype=torch.uint8, device=dev)
    if out_scales is None:
        out_scales = torch.empty((rows, ks // 128), dtype=torch.float16, device=dev)
    _want(out, torch.uint8, (rows, ks // 4), "out")
    _want(out_scales, torch.float16, (rows, ks // 128), "out_scales")
    _check(lib.q2_slice(_ptr(packed), _ptr(scales), n, k, n0, n1, k0, k1, _ptr(out), _ptr(out_scales), _stream()))
    return out, out_scales


def a8_workspace_bytes(m: int, k: int) -> int:
    return int(load().q2_a8_workspace_bytes(m, k))


def q2_linear_a8(x, packed, scales, y=None, workspace=None) -> torch.Tensor:
    """y = s * (c W^T) with x quantised per row to 8-bit codes c and scales s (the codes and scales are left
    in the workspace: bf16 [M, K] at offset 0, f32 [M] after it, 256-byte aligned)."""
    lib = load()
    m, k = x.shape
    n = packed.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed, torch.uint8, (n, k // 4), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    need = a8_workspace_bytes(m, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib.q2_linear_a8(_ptr(x), _ptr(packed), _ptr(scales), _ptr(y), m, n, k, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream()))
    return y


def q4_linear(x, packed4, scale, zero, y=None) -> torch.Tensor:
    """4-bit variant: packed4 u8 [N, K/2] (low nibble = even k), scale / zero f16 [N, K/128]."""
    lib = load()
    m, k = x.shape
    n = packed4.shape[0]
    _want(x, torch.bfloat16, (m, k), "x")
    _want(packed4, torch.uint8, (n, k // 2), "packed4")
    _want(scale, torch.float16, (n, k // 128), "scale")
    _want(zero, torch.float16, (n, k // 128), "zero")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, (m, n), "y")
    _check(lib.q4_linear(_ptr(x), _ptr(packed4), _ptr(scale), _ptr(zero), _ptr(y), m, n, k, _stream()))
    return y


def q2_dequant(packed, scales, w=None) -> torch.Tensor:
    """Test export: float32 [N, K] weights (q - 1) * d."""
    lib = load()
    n, kq = packed.shape
    k = kq * 4
    _want(packed, torch.uint8, (n, kq), "packed")
    _want(scales, torch.float16, (n, k // 128), "scales")
    if w is None:
        w = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    _check(lib.q2_dequant(_ptr(packed), _ptr(scales), _ptr(w), n, k, _stream()))
    return w


def set_dispatch(path: str | None = None, tile: str | None = None, ksplit: int = 0) -> None:
    """Test / profiling control of the launch choice for the whole process (q2_set_dispatch): path None,
    "auto", "gemv" or "gemm"; tile None or a GEMM configuration name; ksplit 0 (automatic), 1 or 2."""
    lib = load()
    _check(lib.q2_set_dispatch(None if path is None else path.encode(), None if tile is None else tile.encode(),
                               int(ksplit)))
