"""The layer norm's exact moments as the kernels compute them, run on the CPU.

tests/host/moments_host.hip builds the kernels' own helpers (csrc/exact_moments.hpp) for
the host and runs the kernels' algorithm on one row: window sums anchored at the row's
largest exponent, exponent bins for the values far below it, and one rounding each of
S1 = sum x and D = K sum x^2 - S1^2 to fp64.  Each result must equal the exact rational
value rounded to nearest, ties to even ("BitNet b1.58: The 1-Bit Ternary LLM Architecture
Guide", "Implementation", Step 2 listing: the layer norm's mean S1 / K and variance
D / K^2, read as exact sums rounded once).  D is checked against the two-pass definition
K sum (x - mean)^2, not against the formula the helpers use.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "moments_host.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def host_moments():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="moments_host_")
    so = os.path.join(d, "moments_host.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-fPIC",
                    "-shared", "-o", so, SRC], check=True)
    lib = ctypes.CDLL(so)
    P = ctypes.c_void_p
    lib.host_moments.argtypes = [P, ctypes.c_int64, P, P, ctypes.POINTER(ctypes.c_int)]
    lib.host_moments.restype = None

    def run(row):
        row = np.ascontiguousarray(row, dtype=np.uint16).reshape(-1)
        out = np.zeros(2, np.float64)
        slow = ctypes.c_int(0)
        lib.host_moments(row.ctypes.data, row.size, out[0:].ctypes.data, out[1:].ctypes.data,
                         ctypes.byref(slow))
        return float(out[0]), float(out[1]), bool(slow.value)
    return run


def _exact(row):
    xs = [Fraction(float(v)) for v in workloads.bf16_bits_to_f32(np.asarray(row, np.uint16))]
    K = len(xs)
    s1 = sum(xs)
    d = K * sum((x - s1 / K) ** 2 for x in xs)
    f = lambda q: q.numerator / q.denominator  # CPython's int division: nearest, ties to even
    return f(s1), f(d)


def _bf(vals):
    return workloads.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _wide(rng, k):
    e = rng.integers(0, 255, size=k)
    return ((rng.integers(0, 2, size=k) << 15) | (e << 7) | rng.integers(0, 128, size=k)).astype(np.uint16)


@pytest.mark.parametrize("k", [1, 2, 7, 64, 1000, 2560, 6912])
def test_fast_path_rows(host_moments, k):
    rng = np.random.default_rng([31, k])
    for row in (_bf(rng.standard_normal(k).astype(np.float32)),
                _bf((40.0 + rng.standard_normal(k)).astype(np.float32)),
                _bf((-3.0 + 0.01 * rng.standard_normal(k)).astype(np.float32)),
                _bf(rng.integers(-5, 6, size=k).astype(np.float32))):
        s1, d, slow = host_moments(row)
        assert not slow
        assert (s1, d) == _exact(row)


@pytest.mark.parametrize("k", [3, 64, 2560, 6912])
def test_slow_path_rows(host_moments, k):
    # exponents over the whole finite range, and Gaussian rows with a twentieth of the
    # values scaled by 2^-50 (below the window)
    rng = np.random.default_rng([32, k])
    rows = [_wide(rng, k) for _ in range(3)]
    x = rng.standard_normal(k).astype(np.float32)
    x[rng.random(k) < 0.05] *= np.float32(2.0 ** -50)
    x[0] = 1.0
    x[-1] = np.float32(2.0 ** -60)
    rows.append(_bf(x))
    for row in rows:
        s1, d, slow = host_moments(row)
        assert slow
        assert (s1, d) == _exact(row)


def test_cancelling_rows(host_moments):
    # x and -x: S1 = 0 exactly, D = K S2; on both paths
    rng = np.random.default_rng(33)
    for half in (_bf(rng.standard_normal(1280).astype(np.float32)), _wide(rng, 1280)):
        row = np.concatenate([half, half ^ np.uint16(0x8000)])
        rng.shuffle(row)
        s1, d, _ = host_moments(row)
        assert s1 == 0.0
        assert (s1, d) == _exact(row)


def test_hand_values(host_moments):
    # 2^20 everywhere but one 2^20 + 2^13: D = (K - 1) 2^26 exactly (K = 4096)
    row = np.full(4096, 2.0 ** 20, np.float32)
    row[1234] += 2.0 ** 13
    assert host_moments(_bf(row))[:2] == (4096 * 2.0 ** 20 + 2.0 ** 13, 4095 * 2.0 ** 26)
    # the extremes of bf16
    assert host_moments(np.array([0x0001, 0x0000], np.uint16))[:2] == (2.0 ** -133, 2.0 ** -266)
    s1, d, _ = host_moments(np.array([0x7F7F, 0xFF7F], np.uint16))
    assert s1 == 0.0 and d == 4 * (255.0 * 2.0 ** 120) ** 2
    # zeros, and a single value (D = 0)
    assert host_moments(np.zeros(16, np.uint16))[:2] == (0.0, 0.0)
    assert host_moments(_bf([-3.5]))[:2] == (-3.5, 0.0)
    # the largest value at the top with a value just inside and just outside the window
    for low, slow in ((2.0 ** -40, False), (2.0 ** -41, True)):
        row = _bf([1.0, low, -low, 1.5])
        s1, d, was_slow = host_moments(row)
        assert was_slow == slow
        assert (s1, d) == _exact(row)


def test_many_equal_terms(host_moments):
    # 2^20 values of the largest magnitude: the 64-bit partial sums are flushed in time
    row = np.full(1 << 20, 0x7F7F, np.uint16)
    row[::3] = 0xFF7F
    assert host_moments(row)[:2] == _exact(row)
