"""The C ABI's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the host code of q2_api.hip and a driver that
calls every entry point with bad, empty and extreme arguments
(tests/abi_sanitize/driver.cpp) are built with the sanitizers on the host side
only (device code is never instrumented), linked with the library's kernel
objects, and run without a GPU: every call must be answered before any HIP
call, with the expected status and no sanitizer report."""
import os
import subprocess

import pytest

from tests.conftest import ROOT
from ternary_weight_quantized_q2_amd import build_lib

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{out}"


def test_abi_validation_under_sanitizers(tmp_path):
    if not os.path.exists(build_lib.HIPCC):
        pytest.fail("hipcc is needed to build the sanitized driver")
    csrc = build_lib.CSRC
    kernel_objs = []
    for name in ("q2_linear.hip", "q2_a8.hip", "q2_pack.hip"):
        obj = os.path.join(build_lib.OBJ_DIR, name + ".o")
        if not os.path.exists(obj):                    # the library build leaves these behind
            build_lib._compile(os.path.join(csrc, name))
        kernel_objs.append(obj)
    api_obj = str(tmp_path / "q2_api_san.o")
    _run([build_lib.HIPCC, *build_lib.FLAGS, *SAN, "-c", os.path.join(csrc, "q2_api.hip"), "-o", api_obj])
    drv_obj = str(tmp_path / "driver.o")
    _run([build_lib.HIPCC, "-O1", "-std=c++17", "-I", build_lib.INCLUDE, *SAN, "-c",
          os.path.join(ROOT, "tests", "abi_sanitize", "driver.cpp"), "-o", drv_obj])
    exe = str(tmp_path / "abi_driver")
    _run([build_lib.HIPCC, "--offload-arch=gfx950", *SAN, drv_obj, api_obj, *kernel_objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi driver ok" in r.stdout, r.stdout + r.stderr
