"""Build libq2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m ternary_weight_quantized_q2_amd.build_lib

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the Python binding loads it.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 instructions anywhere in the device code.
# -amdgpu-mfma-vgpr-form: keep matrix-core results in VGPRs, where the
# per-block rescale reads them, instead of accumulation registers.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


PEAKS_SRC = os.path.join(CSRC, "peaks.hip")          # benchmark-only measurement kernels
PEAKS_LIB = os.path.join(PKG, "libq2_peaks.so")


def build(verbose=True, out=LIB, srcs=None):
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = srcs or sorted(s for s in glob.glob(os.path.join(CSRC, "*.hip")) if s != PEAKS_SRC)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, log in results:
        if log.strip() and verbose:
            print(log, file=sys.stderr)
    tmp = out + ".tmp"
    # -z defs: a symbol left undefined (such as a kernel launch stub that the
    # host compilation pass failed to emit) fails the build instead of the load.
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


def build_peaks(verbose=True):
    """The benchmark's peak-measurement kernels, as a library of their own."""
    return build(verbose=verbose, out=PEAKS_LIB, srcs=[PEAKS_SRC])


if __name__ == "__main__":
    build()
    build_peaks()
