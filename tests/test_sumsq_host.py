"""The RMS norm's exact sum of squares as the kernels compute it, run on the CPU.

tests/host/sumsq_host.hip builds the kernels' own helpers (csrc/exact_sumsq.hpp) for the
host and runs the kernels' algorithm on one row: per-wave anchors (each wave's largest
exponent), 128-bit window sums combined exactly, and, when needed, the general path with
exponent bins for values far below the row's largest; one rounding to fp64.
Each result must equal the exact rational sum rounded to nearest, ties to even ("BitNet
2B4T Guide", "3. Sub-Layer Normalization (SubLN)": the mean square of the row, read as
the exact sum rounded once).  Both the fast path (everything in the window) and the slow
path (bins) are driven, including ties decided only by a value below the window.
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
SRC = os.path.join(ROOT, "tests", "host", "sumsq_host.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def host_sumsq():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="sumsq_host_")
    so = os.path.join(d, "sumsq_host.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-fPIC",
                    "-shared", "-o", so, SRC], check=True)
    lib = ctypes.CDLL(so)
    lib.host_sumsq.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int)]
    lib.host_sumsq.restype = ctypes.c_double

    def run(row):
        row = np.ascontiguousarray(row, dtype=np.uint16).reshape(-1)
        slow = ctypes.c_int(0)
        v = lib.host_sumsq(row.ctypes.data, row.size, ctypes.byref(slow))
        return v, bool(slow.value)
    return run


def _exact(row) -> float:
    vals = workloads.bf16_bits_to_f32(np.asarray(row, np.uint16)).astype(np.float64)
    s = sum(Fraction(float(v)) ** 2 for v in vals)
    return s.numerator / s.denominator  # CPython's int division: nearest, ties to even


def _bf(vals):
    return workloads.to_bf16_bits(np.asarray(vals, dtype=np.float32))


@pytest.mark.parametrize("k", [1, 2, 7, 64, 1000, 2560, 6912])
def test_random_rows_match_exact_sum(host_sumsq, k):
    rng = np.random.default_rng([21, k])
    paths = set()
    for _ in range(40):
        # exponents over a random span: narrow spans stay in the window, wide ones spill
        lo = int(rng.integers(0, 254))
        hi = int(rng.integers(lo, 255))
        e = rng.integers(lo, hi + 1, size=k)
        row = ((rng.integers(0, 2, size=k) << 15) | (e << 7) | rng.integers(0, 128, size=k))
        v, slow = host_sumsq(row.astype(np.uint16))
        assert v == _exact(row), (lo, hi)
        paths.add(slow)
    if k > 1:
        assert paths == {False, True}


def test_gaussian_rows_fast_path(host_sumsq):
    rng = np.random.default_rng(22)
    for scale in (1e-3, 1.0, 3.0, 1e4):
        row = _bf((scale * rng.standard_normal(2560)).astype(np.float32))
        v, slow = host_sumsq(row)
        assert not slow and v == _exact(row)


def test_ties(host_sumsq):
    # in the window: 2^54 + 2 is half way between 2^54 and 2^54 + 4 (fp64 neighbours)
    # and rounds to the even one; 2^54 + 3 rounds up
    assert host_sumsq(_bf([2.0 ** 27, 1.0, 1.0])) == (2.0 ** 54, False)
    assert host_sumsq(_bf([1.0, 1.0, 1.0, 2.0 ** 27])) == (2.0 ** 54 + 4, False)
    # the same sums with the terms in different waves (groups of 8 go to threads in turn,
    # threads 64 apart to the next wave): anchors 2^27 and 2^0 apart by 27 exponents
    # (> 16) take the general path; closer anchors are combined directly
    row = np.zeros(8 * 256, np.float32)
    row[0], row[8 * 64], row[8 * 128] = 2.0 ** 27, 1.0, 1.0
    assert host_sumsq(_bf(row)) == (2.0 ** 54, True)
    row[8 * 192] = 2.0 ** -60
    assert host_sumsq(_bf(row)) == (2.0 ** 54 + 4, True)
    row = np.zeros(8 * 256, np.float32)
    row[0], row[8 * 64], row[8 * 128] = 2.0 ** 8, 2.0 ** -19, 2.0 ** -19
    # 2^16 + 2^-37 is half way between 2^16 and 2^16 + 2^-36: ties to even (the anchors
    # lie 27 exponents apart: the general path)
    assert host_sumsq(_bf(row)) == (2.0 ** 16, True)
    row[8 * 192 + 3] = 2.0 ** -30
    assert host_sumsq(_bf(row)) == (2.0 ** 16 + 2.0 ** -36, True)
    # anchors 14 apart are combined directly, exactly: 2^16 + 2 * 2^-12 + 3 * 2^-2
    row = np.zeros(8 * 256, np.float32)
    row[1], row[8 * 64 + 5], row[8 * 65], row[8 * 128 + 7] = 2.0 ** 8, 2.0 ** -6, 2.0 ** -6, 1.5
    assert host_sumsq(_bf(row)) == (2.0 ** 16 + 2.0 ** -11 + 2.25, False)
    # 2^200 + 2^147 is a tie (ulp 2^148): alone it rounds down to 2^200; a value far below
    # the window (2^50 squares to 2^100, 2^100 below) tips it up through the slow path
    assert host_sumsq(_bf([2.0 ** 100, 2.0 ** 73, 2.0 ** 73])) == (2.0 ** 200, False)
    assert host_sumsq(_bf([2.0 ** 100, 2.0 ** 73, 2.0 ** 50, 2.0 ** 73])) == (2.0 ** 200 + 2.0 ** 148,
                                                                           True)


def test_extremes(host_sumsq):
    # the largest finite bf16 next to the smallest subnormal: the subnormal only matters
    # as a sticky bit, and the sum is the larger square itself (exact in fp64)
    v, slow = host_sumsq(np.array([0x7F7F, 0x0001, 0x8001], np.uint16))
    assert slow and v == 255.0 ** 2 * 2.0 ** 240
    # subnormals alone (E = 0 reads as E' = 1): 0x0001 = 2^-133, 0x0040 = 2^-127
    assert host_sumsq(np.array([0x0001], np.uint16)) == (2.0 ** -266, False)
    assert host_sumsq(np.array([0x0040, 0x8001], np.uint16)) == (2.0 ** -254 + 2.0 ** -266, False)
    # zeros (and signed zeros) add nothing, also below the window
    assert host_sumsq(np.array([0x0000, 0x8000], np.uint16)) == (0.0, False)
    assert host_sumsq(np.array([0x7F00, 0x0000, 0x8000], np.uint16))[1] is False


def test_many_equal_terms_carry(host_sumsq):
    # 2^20 copies of the largest significand at the top of the window: the window sum
    # carries past 64 bits, and the total is exactly 2^20 (255 2^-7)^2
    row = np.full(1 << 20, 0x3FFF, np.uint16)  # 1.9921875
    v, slow = host_sumsq(row)
    assert not slow and v == float(2 ** 20 * Fraction(255, 128) ** 2)

