"""The int4 activation code as the kernels compute it, run on the CPU.

q4 (csrc/common.hpp) replaces the division of each code by the row's scale with a product
by its reciprocal, and divides only where the product lies within 2^-18 of a half-integer
("BitNet a4.8 Guide", "1. Hybrid W1.58 / A4 Quantization Function": q = Clip(Round(x / s),
-8, 7), s = a / 7).  tests/host/q4_host.hip builds the same function for the host and
compares it with one IEEE division per code, over every finite bf16 value within the
absmax, and over fp32 values on and around each quotient k + 1/2, for absmax values across
the fp32 range (the smallest ones, where the reciprocal overflows, included)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "q4_host.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def check():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="q4_host_")
    so = os.path.join(d, "q4_host.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-fPIC",
                    "-ffp-contract=off", "-shared", "-o", so, SRC], check=True)
    lib = ctypes.CDLL(so)
    lib.host_q4_check.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.host_q4_check.restype = None

    def run(amax):
        amax = np.ascontiguousarray(amax, dtype=np.float32)
        counts = np.zeros(3, np.uint64)
        lib.host_q4_check(amax.ctypes.data, amax.size, counts.ctypes.data)
        return [int(c) for c in counts]
    return run


def test_q4_matches_the_division(check):
    rng = np.random.default_rng(51)
    amax = np.concatenate([
        rng.uniform(0.5, 40.0, 200),                        # typical activation rows
        np.exp2(rng.uniform(-120, 120, 200)),               # across the fp32 range
        [1e-5, 1.0, 7.0, 3.5, 2.0 ** -126, 1e-38, 1e-45],   # eps, exact quotients, tiny
        workloads_bf16(rng),                                # bf16 maxima (the kernels' case)
    ]).astype(np.float32)
    compared, bad, band = check(amax)
    assert compared > 5_000_000
    assert bad == 0
    # the exact-division band was exercised (the half-integer neighbourhoods), and is rare
    # among the bf16 values
    assert band > 1000


def workloads_bf16(rng):
    import workloads
    x = rng.standard_normal(300).astype(np.float32) * np.float32(4.0)
    return np.abs(workloads.bf16_bits_to_f32(workloads.to_bf16_bits(x))) + np.float32(2.0 ** -20)
