"""GPU parity of the backward pass under the straight-through estimators
(bitlinear_backward) against the oracle's float64 gradients.

int8 codes: "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "Implementation"
(Step 1 quantizers pass gradients straight through; Step 2 forward); int4 codes: "BitNet
a4.8 Guide", "Implementation" (Step 2 quantizers with the clipping masks; Step 3 forward).

Two kinds of inputs:
- exact: dY = j / 16 with |j| <= 8, power-of-two scales, gamma = 0.75.  Every product and
  partial sum is then exact in fp32 whatever the order, so the kernels must return the
  oracle's value rounded to fp32, to the bit -- a strict check of indexing, transposes,
  padding, the three-part split and the split-k fixup.
- random: bf16 dY, random scales and codes.  The fp32 accumulation then rounds; the bound
  is the classical one for a sum of n terms in any order, (n + 8) 2^-24 sum |terms| (n
  the contraction length after padding and splitting), with the sum of |terms| computed
  in float64 from the same operands.  A dropped or misplaced term breaks it at these
  sizes, and the exact cases pin the structure to the bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, say, to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _unpack_2bit(packed: np.ndarray, K: int) -> np.ndarray:
    fields = np.stack([(packed >> (2 * j)) & 3 for j in range(4)], axis=-1)
    return fields.reshape(packed.shape[0], K).astype(np.int64) - 1


def _codes(xq: np.ndarray, bits: int, K: int) -> np.ndarray:
    if bits == 8:
        return xq.astype(np.int64)
    lo = (xq & 0xF).astype(np.int64)
    hi = (xq >> 4).astype(np.int64)
    v = np.stack([lo, hi], axis=-1).reshape(xq.shape[0], K)
    return np.where(v >= 8, v - 16, v)


def _pack(fields: np.ndarray) -> np.ndarray:
    return (fields[:, 0::4] | (fields[:, 1::4] << 2) | (fields[:, 2::4] << 4) |
            (fields[:, 3::4] << 6)).astype(np.uint8)


def _case(M, N, K, bits, gran, seed, exact):
    """Seeded operands of the backward: dY bits, codes, scales, gamma, packed weights."""
    rng = np.random.default_rng([seed, M, N, K, bits, gran, exact])
    packed = _pack(rng.integers(0, 3, (N, K)).astype(np.uint8))
    if bits == 8:
        xq = rng.integers(-128, 128, (M, K)).astype(np.int8)
    else:
        xq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    ns = M if gran == oracle.PER_TOKEN else 1
    if exact:
        dY = workloads.to_bf16_bits((rng.integers(-8, 9, (M, N)) / 16.0).astype(np.float32))
        e = rng.integers(-2, 3, ns).astype(np.float32)
        s = (np.float32(0.75) * np.exp2(e) if bits == 8 else np.exp2(e)).astype(np.float32)
        g = np.float32(0.75)
    else:
        dY = workloads.to_bf16_bits((0.01 * rng.standard_normal((M, N))).astype(np.float32))
        s = ((rng.random(ns) + 0.5) * (0.02 if bits == 8 else 0.3)).astype(np.float32)
        g = np.float32(0.0125 + 0.01 * rng.random())
    return dY, xq, s, g, packed


def _run(dY, xq, s, g, packed, bits, gran, X=None, W=None, want=("dX", "dW", "dbias")):
    d = bl.backward(to_dev(dY), to_dev(xq), to_dev(s), to_dev(packed), to_dev(np.array([g])),
                    bits=bits, gran=gran, X=None if X is None else to_dev(X),
                    W=None if W is None else to_dev(W), want=want)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in d.items()}


def _abs_terms(dY, xq, s, g, packed, bits, gran, K, rows=None, cols=None):
    """sum of |terms| of each dX (rows of dY) and dW (columns of dY) entry, float64."""
    dy = np.abs(workloads.bf16_bits_to_f32(dY).astype(np.float64))
    srow = np.broadcast_to(np.asarray(s, np.float64), (dY.shape[0],))
    q = np.abs(_codes(xq, bits, K)).astype(np.float64)
    fx = (np.float64(g) / srow) if bits == 8 else np.full_like(srow, np.float64(g))
    fw = (np.float64(g) / srow) if bits == 8 else srow
    out = {}
    dyr = dy if rows is None else dy[rows]
    out["dX"] = (dyr * (fx if rows is None else fx[rows])[:, None]) @ np.abs(_unpack_2bit(packed, K))
    dyc = dy if cols is None else dy[:, cols]
    out["dW"] = (dyc * fw[:, None]).T @ q
    return out


def _assert_close(got, ref, terms, n, what):
    tol = (n + 8) * U * terms + 1e-37
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d beyond (n+8) 2^-24 sum|terms| (n=%d), worst err %.3g tol %.3g" % (
        what, int(bad.sum()), bad.size, n, float(err[bad].max()), float(tol[bad][np.argmax(err[bad])]))


def _assert_exact(got, ref, what):
    assert_same_bytes(got.astype(np.float32), ref.astype(np.float32), what)


def _pad32(v):
    return (v + 31) // 32 * 32


# (M, N, K): one tile; ragged M, N (dY rows padded), K not a multiple of 64; several tiles;
# a single tile split in k (dX: 1 tile, 32 k steps; dW: 4 tiles, 24 k steps); tiny
SHAPES = [(8, 512, 256), (300, 260, 272), (513, 520, 640), (256, 1024, 256), (1, 1, 16),
          (33, 96, 48)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("gran", [oracle.PER_TOKEN, oracle.PER_TENSOR])
def test_backward_exact(M, N, K, bits, gran):
    dY, xq, s, g, packed = _case(M, N, K, bits, gran, 0, exact=True)
    say("backward exact", dict(M=M, N=N, K=K, bits=bits, gran=gran))
    got = _run(dY, xq, s, g, packed, bits, gran)
    ref = oracle.backward(dY, xq, bits, s, gran, packed, g)
    for k in ("dX", "dW", "dbias"):
        _assert_exact(got[k], ref[k], "%s exact" % k)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("gran", [oracle.PER_TOKEN, oracle.PER_TENSOR])
def test_backward_random(M, N, K, bits, gran):
    dY, xq, s, g, packed = _case(M, N, K, bits, gran, 1, exact=False)
    say("backward random", dict(M=M, N=N, K=K, bits=bits, gran=gran))
    got = _run(dY, xq, s, g, packed, bits, gran)
    ref = oracle.backward(dY, xq, bits, s, gran, packed, g)
    t = _abs_terms(dY, xq, s, g, packed, bits, gran, K)
    _assert_close(got["dX"], ref["dX"], t["dX"], _pad32(N) + 16, "dX")
    _assert_close(got["dW"], ref["dW"], t["dW"], 3 * _pad32(M) + 16, "dW")
    # fp64 column sums rounded once: within one fp32 rounding of the exact sum
    np.testing.assert_allclose(got["dbias"], ref["dbias"], rtol=2 * U, atol=1e-37)


def _mask_inputs(M, N, K, rng, s):
    """X with x / s on and just past the clipping edges -8 and 7 (s a power of two, so
    the quotient is exact), W with |w| on and just past 1.5."""
    v = rng.uniform(-10.0, 9.0, (M, K)).astype(np.float32)
    edges = np.array([-8.0, 7.0, -8.000001, 7.000001, -7.999999, 6.999999, 0.0], np.float32)
    v.reshape(-1)[: edges.size * 3] = np.tile(edges, 3)
    X = (v * np.asarray(s, np.float32).reshape(-1, 1)).astype(np.float32)
    W = rng.uniform(-2.0, 2.0, (N, K)).astype(np.float32)
    wedges = np.array([1.5, -1.5, 1.5000001, -1.5000001, 1.4999999], np.float32)
    W.reshape(-1)[: wedges.size * 2] = np.tile(wedges, 2)
    return X, W


@pytest.mark.parametrize("M,N,K", [(300, 260, 272), (256, 1024, 256)])
@pytest.mark.parametrize("gran", [oracle.PER_TOKEN, oracle.PER_TENSOR])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_int4_masks(M, N, K, gran, dtype):
    dY, xq, s, g, packed = _case(M, N, K, 4, gran, 2, exact=True)
    rng = np.random.default_rng([3, M, N, K])
    X, W = _mask_inputs(M, N, K, rng, s)
    if dtype == "bf16":
        X, W = workloads.to_bf16_bits(X), workloads.to_bf16_bits(W)
    say("backward int4 masks", dict(M=M, N=N, K=K, gran=gran, dtype=dtype))
    got = _run(dY, xq, s, g, packed, 4, gran, X=X, W=W)
    ref = oracle.backward(dY, xq, 4, s, gran, packed, g, X=X, W=W)
    free = oracle.backward(dY, xq, 4, s, gran, packed, g, want=("dX", "dW"))
    for k in ("dX", "dW", "dbias"):
        _assert_exact(got[k], ref[k], "%s masked" % k)
    # both masks actually cut something, and left most entries alone
    for k in ("dX", "dW"):
        cut = (ref[k] == 0) & (free[k] != 0)
        assert 0 < cut.mean() < 0.5, (k, cut.mean())


def test_backward_int8_ignores_masks():
    M, N, K = 64, 96, 128
    dY, xq, s, g, packed = _case(M, N, K, 8, oracle.PER_TOKEN, 4, exact=True)
    X, W = _mask_inputs(M, N, K, np.random.default_rng(5), np.exp2(np.zeros(M, np.float32)))
    say("backward int8 with X, W given")
    a = _run(dY, xq, s, g, packed, 8, oracle.PER_TOKEN, X=X * 100, W=W * 100)
    b = _run(dY, xq, s, g, packed, 8, oracle.PER_TOKEN)
    for k in a:
        assert_same_bytes(a[k], b[k], k)


@pytest.mark.parametrize("want", [("dX",), ("dW",), ("dbias",), ("dX", "dbias")])
def test_backward_partial_outputs(want):
    M, N, K = 300, 260, 272
    dY, xq, s, g, packed = _case(M, N, K, 8, oracle.PER_TOKEN, 6, exact=True)
    say("backward outputs", want)
    got = _run(dY, xq, s, g, packed, 8, oracle.PER_TOKEN, want=want)
    ref = oracle.backward(dY, xq, 8, s, oracle.PER_TOKEN, packed, g, want=want)
    assert set(got) == set(want)
    for k in want:
        _assert_exact(got[k], ref[k], k)


def test_backward_zero_dy_and_deterministic():
    M, N, K = 513, 520, 640
    dY, xq, s, g, packed = _case(M, N, K, 8, oracle.PER_TOKEN, 7, exact=False)
    say("backward zero dY / determinism")
    z = _run(np.zeros_like(dY), xq, s, g, packed, 8, oracle.PER_TOKEN)
    for k, v in z.items():
        assert (v == 0).all(), k
    a = _run(dY, xq, s, g, packed, 8, oracle.PER_TOKEN)
    b = _run(dY, xq, s, g, packed, 8, oracle.PER_TOKEN)
    for k in a:
        assert_same_bytes(a[k], b[k], k + " (repeat)")


def _sampled(M, N, K, bits, gran, exact, rows, cols, seed):
    dY, xq, s, g, packed = _case(M, N, K, bits, gran, seed, exact=exact)
    say("backward sampled", dict(M=M, N=N, K=K, bits=bits, gran=gran, exact=exact))
    got = _run(dY, xq, s, g, packed, bits, gran)
    sr = s[rows] if gran == oracle.PER_TOKEN else s
    # rows of dX need only those rows of dY; rows of dW only those columns of dY
    ref_x = oracle.backward(dY[rows], xq[rows], bits, sr, gran, packed, g, want=("dX",))["dX"]
    ref_w = oracle.backward(np.ascontiguousarray(dY[:, cols]), xq, bits, s, gran, packed[cols], g,
                            want=("dW", "dbias"))
    if exact:
        _assert_exact(got["dX"][rows], ref_x, "dX rows")
        _assert_exact(got["dW"][cols], ref_w["dW"], "dW rows")
        _assert_exact(got["dbias"][cols], ref_w["dbias"], "dbias")
    else:
        tx = _abs_terms(dY, xq, s, g, packed, bits, gran, K, rows=rows)["dX"]
        tw = _abs_terms(dY, xq, s, g, packed, bits, gran, K, cols=cols)["dW"]
        _assert_close(got["dX"][rows], ref_x, tx, _pad32(N) + 16, "dX rows")
        _assert_close(got["dW"][cols], ref_w["dW"], tw, 3 * _pad32(M) + 16, "dW rows")
        np.testing.assert_allclose(got["dbias"][cols], ref_w["dbias"], rtol=2 * U, atol=1e-37)


# 2B-shaped layers at the prefill batch: dX runs 80 tiles split in k (up) or 216 whole
# tiles (down); dW 270 tiles, 256 whole and 14 split (rows 3328.. of the last column block)
@pytest.mark.parametrize("N,K", [workloads.SHAPE_UP[::-1], workloads.SHAPE_DOWN[::-1]])
@pytest.mark.parametrize("exact", [True, False])
def test_backward_2b_prefill_sampled(N, K, exact):
    M = 2048
    rows = np.array([0, 1, 255, 256, 1000, 2047])
    cols = np.array([0, 31, 32, 255, 3328, 4000, N - 1]) if N > 4000 else np.array([0, 31, 1000, N - 1])
    _sampled(M, N, K, 8, oracle.PER_TOKEN, exact, rows, cols, seed=8)


def test_backward_70b_int4_sampled():
    M, N, K = 4096, workloads.SHAPE_70B[1], workloads.SHAPE_70B[0]
    _sampled(M, N, K, 4, oracle.PER_TOKEN, True, np.array([0, 4095]), np.array([0, 28671]), seed=9)
