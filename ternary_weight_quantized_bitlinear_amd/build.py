"""Build libbitlinear.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every translation unit is compiled with:
  -O3 --offload-arch=gfx950        CDNA4 code only
  -ffp-contract=off                 no a*b+c -> fma contraction (the rescale is two
                                    separately rounded fp32 operations)
  -fhip-fp32-correctly-rounded-divide-sqrt
                                    fp32 division rounds correctly (scales, gamma/s)
  -fno-gpu-flush-denormals-to-zero  subnormal fp32 values are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed-fp32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbitlinear.so")
# matrix-core calibration loops for the benchmark (not part of the BitLinear C ABI)
CALIB_LIB = os.path.join(PKG, "libbitlinear_calib.so")
CALIB_SOURCES = ["calib.hip"]
SOURCES = ["api.hip", "wquant.hip", "aquant.hip", "gemv.hip", "gemm.hip", "gemm_big.hip", "gemm_mid.hip",
           "gemm_f6f4.hip", "norm.hip", "gemm_bf16.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD_DIR, extra=()) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds.  `extra`
    flags go to every compile (the host-sanitizer build of the tests uses them)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    if out == LIB:
        _link(CALIB_LIB, [_compile(src, build_dir, extra) for src in CALIB_SOURCES])
        if verbose:
            print("built", CALIB_LIB)
    return out


def _link(out: str, objs) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
