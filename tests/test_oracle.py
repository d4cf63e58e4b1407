"""Pins of the CPU oracle against what the pages and mathematics fix.

No GPU.  Each test checks the oracle against something other than itself:
hand-worked examples (tests/golden), exact rational arithmetic (tests/exact.py),
a library matmul, closed forms, invariants and textbook statistics.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact import f32_bits, f32_from_bits, frac_of_f32, round_half_even, round_to_f32

EPS = np.float32(1e-5)


def _bits(h):
    return int(h, 16)


def _unpack_2bit(packed: np.ndarray, K: int) -> np.ndarray:
    """Documented layout: field (c+1) of code k in bits 2*(k%4) of byte k/4."""
    fields = np.stack([(packed >> (2 * j)) & 3 for j in range(4)], axis=-1)
    return fields.reshape(packed.shape[0], K).astype(np.int64) - 1


def _unpack_nibbles(xq: np.ndarray, K: int) -> np.ndarray:
    lo = (xq & 0xF).astype(np.int64)
    hi = (xq >> 4).astype(np.int64)
    v = np.stack([lo, hi], axis=-1).reshape(xq.shape[0], K)
    return np.where(v >= 8, v - 16, v)


# ---------------------------------------------------------------- worked examples

def test_worked_weights(golden):
    g = golden["weights"]
    W = np.array(g["W"], np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)
    assert f32_bits(gamma) == _bits(g["gamma_bits"])
    assert codes.tolist() == g["codes"]
    assert packed.tolist() == g["packed"]


@pytest.mark.parametrize("name", ["B", "C", "D", "E"])
def test_worked_acts_and_forward(golden, name):
    ex = [e for e in golden["acts"] if e["name"] == name][0]
    W = np.array(golden["weights"]["W"], np.float32)
    packed, gamma, _ = oracle.quantize_weights(W)
    x = np.array([ex["x"]], np.float32)
    bits = ex["bits"]
    xq, s = oracle.quantize_acts(x, bits=bits)
    assert f32_bits(s[0]) == _bits(ex["scale_bits"])
    if bits == 8:
        assert xq[0].tolist() == ex["q"]
    else:
        assert xq[0].tolist() == ex["packed_bytes"]
        assert _unpack_nibbles(xq, 4)[0].tolist() == ex["q"]
    y, acc = oracle.forward(xq, bits, s, oracle.PER_TOKEN, packed, gamma)
    y2, acc2 = oracle.forward(xq, bits, s, oracle.PER_TOKEN, packed, gamma, epi=oracle.EPI_RELU2)
    assert acc[0].tolist() == ex["acc"] and acc2[0].tolist() == ex["acc"]
    if "y" in ex:
        assert y[0].tolist() == ex["y"]
        assert y2[0].tolist() == ex["y_relu2"]
    else:
        assert [f32_bits(v) for v in y[0]] == [_bits(h) for h in ex["y_bits"]]
        assert [f32_bits(v) for v in y2[0]] == [_bits(h) for h in ex["y_relu2_bits"]]


def test_worked_per_tensor(golden):
    ex = golden["per_tensor"]
    W = np.array(golden["weights"]["W"], np.float32)
    packed, gamma, _ = oracle.quantize_weights(W)
    X = np.array(ex["X"], np.float32)
    xq, s = oracle.quantize_acts(X, bits=8, gran=oracle.PER_TENSOR)
    assert s.shape == (1,) and f32_bits(s[0]) == _bits(ex["scale_bits"])
    assert xq.tolist() == ex["q"]
    y, acc = oracle.forward(xq, 8, s, oracle.PER_TENSOR, packed, gamma)
    assert acc.tolist() == ex["acc"] and y.tolist() == ex["y"]


def test_worked_zeros(golden):
    z = golden["zeros"]
    W = np.zeros((3, 8), np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)
    assert f32_bits(gamma) == _bits(z["gamma_bits"])
    assert (codes == 0).all() and (packed == z["packed_byte"]).all()
    X = np.zeros((2, 8), np.float32)
    for bits, key in ((8, "int8_scale_bits"), (4, "int4_scale_bits")):
        xq, s = oracle.quantize_acts(X, bits=bits)
        assert all(f32_bits(v) == _bits(z[key]) for v in s)
        assert (xq == 0).all()
        Xr = np.random.default_rng(5).standard_normal((2, 8)).astype(np.float32)
        xq2, s2 = oracle.quantize_acts(Xr, bits=bits)
        for epi in (oracle.EPI_NONE, oracle.EPI_RELU2):
            y, acc = oracle.forward(xq2, bits, s2, 0, packed, gamma, epi=epi)
            assert (acc == 0).all() and (y == 0).all()


# ---------------------------------------------------------------- gamma = exact mean

def _exact_mean_f32(W: np.ndarray) -> np.float32:
    total = sum((abs(frac_of_f32(v)) for v in W.ravel()), Fraction(0))
    return round_to_f32(total / W.size)


@pytest.mark.parametrize("seed", range(6))
def test_gamma_is_correctly_rounded_mean(seed):
    rng = np.random.default_rng(seed)
    n, k = 7, 12
    kind = seed % 3
    if kind == 0:
        W = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    elif kind == 1:  # wide exponent range
        W = (rng.standard_normal((n, k)) * 2.0 ** rng.integers(-60, 60, (n, k))).astype(np.float32)
    else:  # subnormals and tiny normals mixed with ordinary values
        W = (rng.standard_normal((n, k)) * 2.0 ** rng.integers(-149, -120, (n, k))).astype(
            np.float32)
        W[0, :3] = [1.0, -3.0, 0.25]
    g = oracle.gamma(W)
    ref = max(_exact_mean_f32(W), EPS)
    assert f32_bits(g) == f32_bits(ref)


def test_gamma_ties_to_even():
    # mean = (1 + 2^-24) exactly: the midpoint between 1 and 1 + 2^-23 -> ties to 1.0
    W = np.array([[1.0, 1.0 + 2.0 ** -23]], np.float32)
    assert f32_bits(oracle.gamma(W)) == f32_bits(np.float32(1.0))
    # mean = 1 + 3*2^-24: midpoint between 1+2^-23 and 1+2^-22 -> ties to 1+2^-22 (even)
    W = np.array([[1.0 + 2.0 ** -23, 1.0 + 2.0 ** -22]], np.float32)
    assert f32_bits(oracle.gamma(W)) == f32_bits(np.float32(1.0 + 2.0 ** -22))


def test_gamma_large_sum_exact():
    # 2^20 copies of a value whose fp32 running sum would drift: exact mean is the value
    v = np.float32(0.015958)
    W = np.full((1024, 1024), v, np.float32)
    assert f32_bits(oracle.gamma(W)) == f32_bits(v)
    # mixed magnitudes: exact mean known in closed form
    W = np.zeros((1024, 1024), np.float32)
    W[:, 0] = 3.0
    W[:, 1] = 2.0 ** -30
    exact = (Fraction(3) * 1024 + Fraction(1, 2 ** 30) * 1024) / (1024 * 1024)
    assert f32_bits(oracle.gamma(W)) == f32_bits(round_to_f32(exact))


def test_gamma_eps_clamp():
    W = np.full((2, 4), 1e-7, np.float32)
    assert f32_bits(oracle.gamma(W)) == f32_bits(EPS)
    assert f32_bits(oracle.gamma(W, eps=1e-8)) == f32_bits(np.float32(1e-7))


def test_gamma_bf16_input():
    W = (0.02 * np.random.default_rng(3).standard_normal((16, 32))).astype(np.float32)
    Wb = workloads.to_bf16_bits(W)
    Wf = workloads.bf16_bits_to_f32(Wb)
    assert f32_bits(oracle.gamma(Wb)) == f32_bits(oracle.gamma(Wf))
    pb, gb, cb = oracle.quantize_weights(Wb)
    pf, gf, cf = oracle.quantize_weights(Wf)
    assert (pb == pf).all() and (cb == cf).all()


# ---------------------------------------------------------------- weight codes

def test_weight_codes_threshold_rule():
    """c != 0 exactly when |w| > gamma * (1/2 + 2^-25) (the exact condition for the fp32
    quotient w/gamma to exceed 1/2, which rounds half to even to 0)."""
    rng = np.random.default_rng(11)
    W = (0.02 * rng.standard_normal((8, 64))).astype(np.float32)
    g = oracle.gamma(W)
    # plant boundary values: exactly gamma/2, and its fp32 neighbours
    for _ in range(8):  # replant until gamma no longer moves
        half = np.float32(g) * np.float32(0.5)
        nb = [half, np.nextafter(half, np.float32(1)), np.nextafter(half, np.float32(0)),
              np.nextafter(np.nextafter(half, np.float32(1)), np.float32(1))]
        W[0, :4] = nb
        W[1, :4] = [-v for v in nb]
        g_new = oracle.gamma(W)
        if g_new == g:
            break
        g = g_new
    assert g == oracle.gamma(W) and W[0, 0] == np.float32(g) * np.float32(0.5)
    _, g2, codes = oracle.quantize_weights(W)
    assert f32_bits(g2) == f32_bits(g)
    th = frac_of_f32(g) * (Fraction(1, 2) + Fraction(1, 2 ** 25))
    for (i, j), w in np.ndenumerate(W):
        fw = frac_of_f32(w)
        expect = 0 if abs(fw) <= th else (1 if fw > 0 else -1)
        assert codes[i, j] == expect, (i, j, w)
    # only gamma/2 itself (an exact tie at 0.5) rounds to 0: one ulp above is already past
    # gamma*(1/2 + 2^-25) because ulp(gamma/2) >= gamma*2^-24
    assert codes[0, :4].tolist() == [0, 1, 0, 1] and codes[1, :4].tolist() == [0, -1, 0, -1]


def test_weight_codes_rounding_and_clip():
    """gamma = 32/16 = 2 exactly, so W/gamma hits exact ties: half-to-even, then clip."""
    W = np.array([[1.0, 3.0, 5.0, -1.0, -3.0, -5.0, 0.75, -0.75],
                  [2.0, 2.0, 2.0, 2.0, 2.0, 2.0, 0.25, 0.25]], np.float32)
    packed, g, codes = oracle.quantize_weights(W)
    assert f32_bits(g) == f32_bits(np.float32(2.0))
    # W/gamma = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.375, -0.375] / [1 x6, 0.125 x2]
    assert codes.tolist() == [[0, 1, 1, 0, -1, -1, 0, 0], [1, 1, 1, 1, 1, 1, 0, 0]]


def test_packing_layout_and_field_range():
    W, _ = workloads.parity_layer()
    packed, gamma, codes = oracle.quantize_weights(W)
    N, K = W.shape
    assert packed.shape == (N, K // 4) and packed.nbytes == N * K * 2 // 8
    fields = np.stack([(packed >> (2 * j)) & 3 for j in range(4)])
    assert (fields != 3).all()
    assert (_unpack_2bit(packed, K) == codes).all()
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}


def test_uniform_ternary_roundtrip():
    rng = np.random.default_rng(2)
    W = workloads.ternary_weights(rng, 64, 128)
    packed, gamma, codes = oracle.quantize_weights(W)
    nnz = int(np.count_nonzero(W))
    assert f32_bits(gamma) == f32_bits(round_to_f32(Fraction(nnz, W.size)))
    assert (codes == W.astype(np.int8)).all()


def test_weight_statistics_gaussian():
    """W ~ N(0, s): gamma -> s*sqrt(2/pi); P(c=0) = 2*Phi(sqrt(2/pi)/2) - 1 (textbook)."""
    rng = np.random.default_rng(0)
    s = 0.02
    W = (s * rng.standard_normal((1024, 1024))).astype(np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)
    assert abs(float(gamma) / (s * math.sqrt(2 / math.pi)) - 1) < 3e-3
    p0 = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    frac0 = float(np.mean(codes == 0))
    assert abs(frac0 - p0) < 3e-3
    assert abs(float(np.mean(codes == 1)) - (1 - p0) / 2) < 3e-3


def test_weight_scaling_and_sign_invariance():
    W, _ = workloads.parity_layer()
    p, g, c = oracle.quantize_weights(W)
    pn, gn, cn = oracle.quantize_weights(-W)
    assert f32_bits(gn) == f32_bits(g) and (cn == -c).all()
    for j in (-3, 5):
        ps, gs, cs = oracle.quantize_weights((W * np.float32(2.0 ** j)).astype(np.float32))
        assert (cs == c).all() and (ps == p).all()
        assert f32_bits(gs) == f32_bits(np.float32(g * np.float32(2.0 ** j)))


# ---------------------------------------------------------------- activation codes

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_int8_codes_exact(dtype):
    _, X = workloads.parity_layer()
    if dtype == "bf16":
        Xin = workloads.to_bf16_bits(X)
        X = workloads.bf16_bits_to_f32(Xin)
    else:
        Xin = X
    xq, s = oracle.quantize_acts(Xin, bits=8)
    for m in range(X.shape[0]):
        a = max(np.abs(X[m]).max(), EPS)
        s_ref = round_to_f32(Fraction(127) / frac_of_f32(a))
        assert f32_bits(s[m]) == f32_bits(s_ref)
        assert np.abs(xq[m]).max() == 127
        for k in range(X.shape[1]):
            prod = round_to_f32(frac_of_f32(X[m, k]) * frac_of_f32(s_ref))
            q = max(-128, min(127, round_half_even(frac_of_f32(prod))))
            assert xq[m, k] == q
        # real-arithmetic bound: |q - x*127/a| <= 1/2 + 2^-17 (two fp32 roundings at <= 127)
        err = np.abs(xq[m].astype(np.float64) - X[m].astype(np.float64) * 127.0 / float(a))
        assert err.max() <= 0.5 + 2.0 ** -17


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_int4_codes_exact(dtype):
    _, X = workloads.parity_layer(m=4)
    if dtype == "bf16":
        Xin = workloads.to_bf16_bits(X)
        X = workloads.bf16_bits_to_f32(Xin)
    else:
        Xin = X
    xq, s = oracle.quantize_acts(Xin, bits=4)
    q_all = _unpack_nibbles(xq, X.shape[1])
    assert xq.nbytes == X.shape[0] * X.shape[1] // 2
    for m in range(X.shape[0]):
        a = max(np.abs(X[m]).max(), EPS)
        s_ref = round_to_f32(frac_of_f32(a) / 7)
        assert f32_bits(s[m]) == f32_bits(s_ref)
        assert np.abs(q_all[m]).max() == 7 and q_all[m].min() >= -7
        for k in range(X.shape[1]):
            quo = round_to_f32(frac_of_f32(X[m, k]) / frac_of_f32(s_ref))
            assert q_all[m, k] == max(-8, min(7, round_half_even(frac_of_f32(quo))))


def test_int8_multiply_form_on_rare_values():
    """int8 codes come from the fp32 product x * (127/a) (the multiply form printed in
    the b1.58 eq. 2 and the 2B4T operator), not from x / (a/127): the two differ on rare
    inputs.  Find such inputs in a large sample and check them with exact rationals."""
    rng = np.random.default_rng(123)
    rows_ = []
    for a in rng.uniform(0.5, 40.0, 32).astype(np.float32):
        cand = [a]
        for j in range(0, 127):
            c = np.float32((j + 0.5) * float(a) / 127.0)
            for d in range(-3, 4):
                v = c
                for _ in range(abs(d)):
                    v = np.nextafter(v, np.float32(np.sign(d) * np.inf))
                cand.append(v)
        rows_.append(np.array(cand, np.float32))
    X = np.stack(rows_)
    xq, s = oracle.quantize_acts(X, bits=8)
    a = np.maximum(np.abs(X).max(axis=1, keepdims=True), EPS)
    mul = np.rint(X * (np.float32(127) / a))
    div = np.rint(X / (a / np.float32(127)))
    rows, cols = np.nonzero(mul != div)
    assert len(rows) > 0  # the sample does contain inputs that tell the forms apart
    for m, k in zip(rows, cols):
        prod = round_to_f32(frac_of_f32(X[m, k]) * frac_of_f32(s[m]))
        assert xq[m, k] == round_half_even(frac_of_f32(prod))


def test_int8_ties_and_saturation():
    # a = 127 gives s = 1, so x*s = x: exact half-integers exercise the tie rule
    x = np.array([[127.0, -127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.5, 4.5]],
                 np.float32)
    xq, s = oracle.quantize_acts(x, bits=8)
    assert f32_bits(s[0]) == f32_bits(np.float32(1.0))
    assert xq[0].tolist() == [127, -127, 0, 2, 2, 0, -2, -2, 126, -126, 4, 4]


def test_per_tensor_equals_per_token_with_common_max():
    rng = np.random.default_rng(9)
    X = rng.standard_normal((5, 32)).astype(np.float32)
    X[:, 0] = 10.0  # every row has the same absmax -> identical scales
    for bits in (8, 4):
        a, sa = oracle.quantize_acts(X, bits=bits, gran=oracle.PER_TOKEN)
        b, sb = oracle.quantize_acts(X, bits=bits, gran=oracle.PER_TENSOR)
        assert (a == b).all() and sb.shape == (1,) and (sa == sb[0]).all()


def test_act_symmetry_and_power_of_two_scaling():
    _, X = workloads.parity_layer()
    for bits in (8, 4):
        q, s = oracle.quantize_acts(X, bits=bits)
        qn, sn = oracle.quantize_acts(-X, bits=bits)
        K = X.shape[1]
        dq = (lambda t: t.astype(np.int64)) if bits == 8 else (lambda t: _unpack_nibbles(t, K))
        assert (dq(qn) == -dq(q)).all() and (sn == s).all()
        for j in (-4, 3):
            qs, ss = oracle.quantize_acts((X * np.float32(2.0 ** j)).astype(np.float32), bits=bits)
            assert (qs == q).all()
            expect = s * np.float32(2.0 ** -j) if bits == 8 else s * np.float32(2.0 ** j)
            assert (ss == expect.astype(np.float32)).all()


# ---------------------------------------------------------------- contraction & output

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("shape", [(1, 16, 8), (3, 20, 5), (8, 256, 512), (5, 64, 33)])
def test_contraction_matches_library_matmul(bits, shape):
    M, K, N = shape
    W, X = workloads.random_case(17, M, K, N, n_outliers=2)
    packed, gamma, codes = oracle.quantize_weights(W)
    xq, s = oracle.quantize_acts(X, bits=bits)
    q = xq.astype(np.int64) if bits == 8 else _unpack_nibbles(xq, K)
    ref = np.matmul(q, codes.astype(np.int64).T)
    y, acc = oracle.forward(xq, bits, s, oracle.PER_TOKEN, packed, gamma)
    assert (acc == ref).all()


def test_contraction_brute_force_tiny():
    """Every 4-wide ternary row against every activation row in a small grid."""
    import itertools
    rows = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=4)), np.float32)  # 81 x 4
    W = rows
    packed, gamma, codes = oracle.quantize_weights(W)
    assert (codes == W.astype(np.int8)).all()
    X = np.array([[3.0, -1.0, 0.5, 2.0], [-7.0, 7.0, 1.0, -2.0]], np.float32)
    xq, s = oracle.quantize_acts(X, bits=8)
    y, acc = oracle.forward(xq, 8, s, 0, packed, gamma)
    for m in range(2):
        for n in range(81):
            tot = 0
            for k in range(4):
                tot += int(xq[m, k]) * int(W[n, k])
            assert acc[m, n] == tot


@pytest.mark.parametrize("bits", [8, 4])
def test_output_rescale_exact_rational(bits):
    W, X = workloads.parity_layer()
    bias = np.random.default_rng(4).standard_normal(W.shape[0]).astype(np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)
    xq, s = oracle.quantize_acts(X, bits=bits)
    for b in (None, bias):
        for epi in (0, 1):
            y, acc = oracle.forward(xq, bits, s, 0, packed, gamma, bias=b, epi=epi)
            for m in range(0, X.shape[0], 3):
                fg, fs = frac_of_f32(gamma), frac_of_f32(s[m])
                f = round_to_f32(fg / fs if bits == 8 else fs * fg)
                for n in range(0, W.shape[0], 37):
                    v = round_to_f32(Fraction(int(acc[m, n])) * frac_of_f32(f))
                    if b is not None:
                        v = round_to_f32(frac_of_f32(v) + frac_of_f32(b[n]))
                    if epi:
                        r = max(frac_of_f32(v), Fraction(0))
                        v = round_to_f32(r * r)
                    assert f32_bits(y[m, n]) == f32_bits(v), (m, n)


def test_output_matches_listing_formulation_float64():
    """The listings' F.linear(x_q, w_q) * (gamma / scale): float64 within 1e-6 relative."""
    W, X = workloads.parity_layer()
    packed, gamma, codes = oracle.quantize_weights(W)
    xq, s = oracle.quantize_acts(X, bits=8)
    y, acc = oracle.forward(xq, 8, s, 0, packed, gamma)
    ref = torch.nn.functional.linear(torch.from_numpy(xq.astype(np.float64)),
                                     torch.from_numpy(codes.astype(np.float64)))
    ref = ref * (float(gamma) / torch.from_numpy(s.astype(np.float64))[:, None])
    ref = ref.numpy()
    assert np.all(np.abs(y - ref) <= 1e-6 * np.abs(ref) + 1e-30)
    # and the layer approximates the float64 product X W^T (quantization error, loose)
    full = X.astype(np.float64) @ (codes.astype(np.float64) * float(gamma)).T
    rel = np.linalg.norm(y - full) / np.linalg.norm(full)
    assert rel < 0.05


def test_closed_form_basis_vector():
    """X = a*e_k: q = 127*e_k, acc[:, n] = 127*c[n, k], y = a*gamma*c[n, k] (within fp32)."""
    W, _ = workloads.parity_layer()
    packed, gamma, codes = oracle.quantize_weights(W)
    K = W.shape[1]
    a = np.float32(3.75)
    for k in (0, 17, K - 1):
        X = np.zeros((1, K), np.float32)
        X[0, k] = a
        xq, s = oracle.quantize_acts(X, bits=8)
        assert xq[0, k] == 127 and np.count_nonzero(xq) == 1
        y, acc = oracle.forward(xq, 8, s, 0, packed, gamma)
        assert (acc[0] == 127 * codes[:, k]).all()
        np.testing.assert_allclose(y[0], float(a) * float(gamma) * codes[:, k], rtol=4e-7)


def test_closed_form_constant_weights():
    K, N = 32, 8
    W = np.full((N, K), 0.3, np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)
    assert f32_bits(gamma) == f32_bits(np.float32(0.3)) and (codes == 1).all()
    X = np.random.default_rng(1).standard_normal((3, K)).astype(np.float32)
    xq, s = oracle.quantize_acts(X, bits=8)
    y, acc = oracle.forward(xq, 8, s, 0, packed, gamma)
    assert (acc == xq.astype(np.int64).sum(axis=1, keepdims=True)).all()


def test_output_symmetries_and_permutation():
    W, X = workloads.parity_layer()
    p, g, c = oracle.quantize_weights(W)
    pn, gn, cn = oracle.quantize_weights(-W)
    xq, s = oracle.quantize_acts(X, bits=8)
    y, acc = oracle.forward(xq, 8, s, 0, p, g)
    yn, accn = oracle.forward(xq, 8, s, 0, pn, gn)
    assert (accn == -acc).all() and (yn == -y).all()
    # scaling an activation row by 2^j scales y by exactly 2^j
    Xs = X.copy()
    Xs[2] *= np.float32(8.0)
    xqs, ss = oracle.quantize_acts(Xs, bits=8)
    ys, _ = oracle.forward(xqs, 8, ss, 0, p, g)
    assert (ys[2] == y[2] * np.float32(8.0)).all()
    # permuting the K axis of X and W alike leaves acc unchanged
    perm = np.random.default_rng(8).permutation(W.shape[1])
    pp, gp, cp = oracle.quantize_weights(np.ascontiguousarray(W[:, perm]))
    xqp, sp = oracle.quantize_acts(np.ascontiguousarray(X[:, perm]), bits=8)
    yp, accp = oracle.forward(xqp, 8, sp, 0, pp, gp)
    assert (accp == acc).all() and (yp == y).all()


def test_relu2_closed_form():
    W = np.array([[1.0, 0.0, 0.0, 0.0], [-1.0, 0.0, 0.0, 0.0]], np.float32)
    packed, gamma, codes = oracle.quantize_weights(W)  # gamma = 1/4 -> codes [[1,0,0,0],[-1,..]]
    assert codes.tolist() == [[1, 0, 0, 0], [-1, 0, 0, 0]]
    X = np.array([[2.0, 0.0, 0.0, 0.0]], np.float32)
    xq, s = oracle.quantize_acts(X, bits=8)
    y, acc = oracle.forward(xq, 8, s, 0, packed, gamma, epi=oracle.EPI_RELU2)
    # acc = [127, -127]; f = fl(0.25 / fl(127/2)); y0 = fl(127*f) = 0.5 (exact here)
    assert acc[0].tolist() == [127, -127]
    y_lin, _ = oracle.forward(xq, 8, s, 0, packed, gamma)
    assert y_lin[0, 1] < 0 and y[0, 1] == 0.0
    assert y[0, 0] == np.float32(y_lin[0, 0]) * np.float32(y_lin[0, 0])


def test_forward_at_matches_full():
    W, X = workloads.parity_layer()
    packed, gamma, _ = oracle.quantize_weights(W)
    for bits in (8, 4):
        xq, s = oracle.quantize_acts(X, bits=bits)
        y, acc = oracle.forward(xq, bits, s, 0, packed, gamma, epi=1, y_dtype=oracle.BF16)
        rng = np.random.default_rng(0)
        ms = rng.integers(0, X.shape[0], 50)
        ns = rng.integers(0, W.shape[0], 50)
        ys, accs = oracle.forward_at(xq, bits, s, 0, packed, gamma, ms, ns, epi=1,
                                     y_dtype=oracle.BF16)
        assert (accs == acc[ms, ns]).all() and (ys == y[ms, ns]).all()


def test_bf16_output_rounding_matches_torch():
    rng = np.random.default_rng(21)
    v = (rng.standard_normal(4096) * 10.0 ** rng.integers(-5, 5, 4096)).astype(np.float32)
    # exact ties between two bf16 values, both parities
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], np.uint32)
    v = np.concatenate([v, ties.view(np.float32), np.array([0.0, -0.0, 65504.0], np.float32)])
    ours = oracle.to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_memory_reduction_figures():
    """The a4.8 Step 4 harness sizes: in=1024, out=2048, batch 2, seq 128 -> weights
    fp16 4096 KB -> 512 KB (87.5% cut), activations fp16 512 KB -> 128 KB (75% cut)."""
    rng = np.random.default_rng(0)
    W = workloads.ternary_weights(rng, 2048, 1024)
    packed, _, _ = oracle.quantize_weights(W)
    assert packed.nbytes == 512 * 1024 and 1 - packed.nbytes / (2048 * 1024 * 2) == 0.875
    X = rng.standard_normal((2 * 128, 1024)).astype(np.float32)
    xq, _ = oracle.quantize_acts(X, bits=4)
    assert xq.nbytes == 128 * 1024 and 1 - xq.nbytes / (256 * 1024 * 2) == 0.75


def test_oracle_rejects_bad_input():
    with pytest.raises(oracle.OracleError):
        oracle.quantize_weights(np.array([[np.inf, 1.0, 0.0, 0.0]], np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.quantize_acts(np.array([[np.nan, 1.0]], np.float32))


# ---------------------------------------------------------------- RMS norm glue
# Pins of the residual + RMS-norm glue between BitLinear layers ("BitNet 2B4T
# Guide", "3. Sub-Layer Normalization (SubLN)"): closed forms and invariants.

def _bf(vals):
    return workloads.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _f(bits):
    return workloads.bf16_bits_to_f32(bits)


def test_rmsnorm_constant_row_is_unit():
    # x = c everywhere: rms = |c|, h = c / sqrt(c^2 + eps) -> 1.0 once rounded to bf16
    X = _bf(np.full((3, 64), [[2.0], [-0.5], [8.0]], dtype=np.float32))
    _, h = oracle.rmsnorm(X)
    assert np.array_equal(_f(h), np.sign(_f(X)))


def test_rmsnorm_single_spike_is_sqrt_k():
    # one nonzero a in K = 16: rms = |a| / 4, h = sign(a) * 4 exactly (eps is negligible)
    x = np.zeros((2, 16), np.float32)
    x[0, 5] = 3.0
    x[1, 11] = -0.375
    _, h = oracle.rmsnorm(_bf(x))
    hf = _f(h)
    assert hf[0, 5] == 4.0 and hf[1, 11] == -4.0
    assert np.count_nonzero(hf) == 2


def test_rmsnorm_power_of_two_scaling_invariant():
    rng = np.random.default_rng(5)
    X = _bf(rng.standard_normal((4, 256)).astype(np.float32))
    _, h0 = oracle.rmsnorm(X, eps=1e-30)
    for j in (-3, 2, 5):
        Xs = _bf(_f(X) * np.float32(2.0 ** j))
        _, hj = oracle.rmsnorm(Xs, eps=1e-30)
        assert np.array_equal(hj, h0), j


def test_rmsnorm_sign_symmetry():
    rng = np.random.default_rng(6)
    X = _bf(rng.standard_normal((3, 128)).astype(np.float32))
    _, h = oracle.rmsnorm(X)
    _, hn = oracle.rmsnorm(_bf(-_f(X)))
    assert np.array_equal(_f(hn), -_f(h))


def test_rmsnorm_output_has_unit_mean_square():
    rng = np.random.default_rng(7)
    X = _bf((3.0 * rng.standard_normal((8, 2560))).astype(np.float32))
    _, h = oracle.rmsnorm(X)
    ms = (_f(h).astype(np.float64) ** 2).mean(axis=1)
    # each h is within half a bf16 ulp (2^-9 relative) of x / rms
    assert np.all(np.abs(ms - 1.0) < 2 * 2.0 ** -8)


def test_rmsnorm_residual_add_rounds_to_bf16():
    # sums chosen so the exact sum is known: 1 + 2^-8 rounds to 1 (tie to even),
    # 1 + 3*2^-8 to 1 + 2^-6 (tie to even), 3 + 0.5 = 3.5 exactly
    x = _bf([[1.0, 1.0, 3.0, -2.0]])
    d = _bf([[2.0 ** -8, 3 * 2.0 ** -8, 0.5, 2.0]])
    x_out, _ = oracle.rmsnorm(x, d)
    assert list(_f(x_out)[0]) == [1.0, 1.0 + 2.0 ** -6, 3.5, 0.0]
    # delta = None is delta = 0
    X = _bf(np.random.default_rng(8).standard_normal((2, 32)).astype(np.float32))
    a = oracle.rmsnorm(X)
    b = oracle.rmsnorm(X, np.zeros_like(X))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rmsnorm_eps_dominates_zero_row():
    # x = 0: h = 0 (no division by zero); tiny x: eps bounds the gain at 1/sqrt(eps)
    X = np.zeros((1, 32), np.uint16)
    _, h = oracle.rmsnorm(X)
    assert not h.any()
    x = _bf(np.full((1, 32), 2.0 ** -20, np.float32))
    _, h = oracle.rmsnorm(x, eps=1e-6)
    assert np.all(_f(h) < 2.0 ** -20 * 1000.0 * 1.01)


def _exact_sumsq(bits_row) -> float:
    """sum of squares in exact rational arithmetic, rounded once to fp64 (CPython's
    int / int division rounds to nearest, ties to even)."""
    s = sum(Fraction(float(v)) ** 2 for v in _f(np.asarray(bits_row, np.uint16)))
    return s.numerator / s.denominator


def _wide_bf16_rows(rng, m, k):
    """bf16 bit patterns with exponents over the whole finite range (subnormals and
    zeros included), random signs and significands."""
    e = rng.integers(0, 255, size=(m, k))
    mant = rng.integers(0, 128, size=(m, k))
    sign = rng.integers(0, 2, size=(m, k))
    return ((sign << 15) | (e << 7) | mant).astype(np.uint16)


@pytest.mark.parametrize("k", [1, 3, 16, 64, 2560])
def test_rmsnorm_sum_of_squares_exact(k):
    # S = sum x'^2 exactly, rounded once: rows spanning the whole exponent range, rows
    # spanning a narrow one (Gaussian), and rows of subnormals
    rng = np.random.default_rng([11, k])
    rows = list(_wide_bf16_rows(rng, 4, k))
    rows.append(_bf(rng.standard_normal(k).astype(np.float32)))
    rows.append((rng.integers(0, 128, size=k) | (rng.integers(0, 2, size=k) << 15)).astype(np.uint16))
    for row in rows:
        assert oracle.sumsq(row) == _exact_sumsq(row)


def test_rmsnorm_sum_of_squares_hand_ties():
    # worked by hand: 2^54 + 2 lies half way between the fp64 neighbours 2^54 and
    # 2^54 + 4 and rounds to the even one, 2^54; any positive remainder tips it up;
    # 2^54 + 3 is past the half way point.  (A running fp64 sum gives 2^54 for all
    # three: each 1 is below half an ulp of 2^54.)
    assert oracle.sumsq(_bf([2.0 ** 27, 1.0, 1.0])) == 2.0 ** 54
    assert oracle.sumsq(_bf([1.0, 2.0 ** 27, 1.0, 2.0 ** -60])) == 2.0 ** 54 + 4
    assert oracle.sumsq(_bf([1.0, 1.0, 1.0, 2.0 ** 27])) == 2.0 ** 54 + 4
    # the extremes of bf16: the smallest subnormal 2^-133 squares to 2^-266; the largest
    # finite value (2 - 2^-7) 2^127 squares to 255^2 2^240, both exact in fp64
    assert oracle.sumsq(np.array([0x0001], np.uint16)) == 2.0 ** -266
    assert oracle.sumsq(np.array([0x7F7F, 0xFF7F], np.uint16)) == 2 * 255.0 ** 2 * 2.0 ** 240
    # the subnormal significand has no hidden bit: 0x0040 is 2^-127
    assert oracle.sumsq(np.array([0x0040, 0x8040], np.uint16)) == 2 * 2.0 ** -254
    assert oracle.sumsq(np.zeros(7, np.uint16)) == 0.0


def test_rmsnorm_h_from_the_exact_sum():
    # h = bf16(fl32(x' r)), r = 1 / sqrt(S / K + eps), recomputed from the exact S
    rng = np.random.default_rng(12)
    X = np.concatenate([_wide_bf16_rows(rng, 3, 96) & np.uint16(0xBFFF),  # |x| < 2^1
                        _bf((0.3 * rng.standard_normal((3, 96))).astype(np.float32))])
    eps = np.float32(1e-6)
    _, h = oracle.rmsnorm(X, eps=float(eps))
    for i in range(X.shape[0]):
        S = _exact_sumsq(X[i])
        r = 1.0 / math.sqrt(S / 96 + float(eps))
        prod = (_f(X[i]).astype(np.float64) * r).astype(np.float32)
        assert np.array_equal(h[i], _bf(prod)), i


# ---------------------------------------------------------------- layer norm
# Pins of the non-affine layer norm before the quantizer ("BitNet b1.58: The 1-Bit
# Ternary LLM Architecture Guide", "Implementation", Step 2 listing): exact rational
# sums, the two-pass definition of the variance, closed forms, invariants, and the
# library layer norm.

def _exact_moments(bits_row):
    """(S1 exact, K * sum (x - S1/K)^2 exact) as Fractions: the sum, and K^2 times the
    variance taken by its two-pass definition."""
    xs = [Fraction(float(v)) for v in _f(np.asarray(bits_row, np.uint16))]
    K = len(xs)
    s1 = sum(xs)
    mean = s1 / K
    return s1, K * sum((x - mean) ** 2 for x in xs)


def _to_f64(fr: Fraction) -> float:
    return fr.numerator / fr.denominator  # int / int: nearest fp64, ties to even


def test_layernorm_constant_row_is_zero():
    # x = c everywhere: the mean is c, every deviation exactly 0, h = +0
    X = _bf(np.full((5, 48), [[2.0], [-0.5], [3.0e38], [2.0 ** -130], [-7.0]], dtype=np.float32))
    _, h = oracle.layernorm(X)
    assert not h.any()


def test_layernorm_two_level_rows_are_plus_minus_one():
    # a row of a (K/2 times) and b (K/2 times): mean (a+b)/2, deviations +-(b-a)/2,
    # variance ((b-a)/2)^2, so h = sign(x - mean) once eps is negligible
    rows = []
    for a, b in [(1.0, 3.0), (-5.0, 2.5), (1000.0, 1008.0), (2.0 ** -10, 2.0 ** -9)]:
        r = np.full(32, a, np.float32)
        r[np.random.default_rng(int(abs(a) + 7)).permutation(32)[:16]] = b
        rows.append(r)
    X = _bf(np.stack(rows))
    _, h = oracle.layernorm(X, eps=1e-30)
    x = _f(X).astype(np.float64)
    assert np.array_equal(_f(h), np.sign(x - x.mean(axis=1, keepdims=True)))


def test_layernorm_worked_example():
    # x = (1, 2, 3, 4): mean 5/2, variance 5/4, h = (x - 5/2) / sqrt(5/4 + eps)
    _, h = oracle.layernorm(_bf([[1.0, 2.0, 3.0, 4.0]]), eps=1e-5)
    want = (np.array([-1.5, -0.5, 0.5, 1.5]) / math.sqrt(1.25 + float(np.float32(1e-5))))
    assert np.array_equal(h[0], _bf(want.astype(np.float32)))
    assert list(_f(h[0])) == [-1.34375, -229 / 512, 229 / 512, 1.34375]


def test_layernorm_shift_invariant():
    # integer rows and integer shifts stay exact in bf16; with K = 64 the mean is a short
    # dyadic number, so every deviation, the variance and h are unchanged by the shift
    rng = np.random.default_rng(21)
    X = rng.integers(-60, 60, size=(4, 64)).astype(np.float32)
    _, h0 = oracle.layernorm(_bf(X))
    for c in (-100.0, 37.0, 150.0):
        _, hc = oracle.layernorm(_bf(X + np.float32(c)))
        assert np.array_equal(hc, h0), c


def test_layernorm_power_of_two_scaling_invariant():
    rng = np.random.default_rng(22)
    X = _bf((1.0 + rng.standard_normal((4, 256))).astype(np.float32))
    _, h0 = oracle.layernorm(X, eps=1e-30)
    for j in (-3, 2, 5):
        _, hj = oracle.layernorm(_bf(_f(X) * np.float32(2.0 ** j)), eps=1e-30)
        assert np.array_equal(hj, h0), j


def test_layernorm_sign_symmetry():
    rng = np.random.default_rng(23)
    X = _bf((0.5 + rng.standard_normal((3, 128))).astype(np.float32))
    _, h = oracle.layernorm(X)
    _, hn = oracle.layernorm(_bf(-_f(X)))
    assert np.array_equal(_f(hn), -_f(h))


@pytest.mark.parametrize("k", [1, 2, 3, 16, 64, 2560])
def test_layernorm_sums_exact(k):
    # fp64(S1) and fp64(D) against exact rational arithmetic, D by the two-pass
    # definition K * sum (x - mean)^2: whole-range rows, Gaussian rows around an offset,
    # subnormal rows, and rows whose terms cancel
    rng = np.random.default_rng([24, k])
    rows = list(_wide_bf16_rows(rng, 4, k))
    rows.append(_bf((5.0 + rng.standard_normal(k)).astype(np.float32)))
    rows.append((rng.integers(0, 128, size=k) | (rng.integers(0, 2, size=k) << 15)).astype(np.uint16))
    half = _wide_bf16_rows(rng, 1, (k + 1) // 2)[0]
    rows.append(np.concatenate([half, half ^ np.uint16(0x8000)])[:k])
    for row in rows:
        s1, d = _exact_moments(row)
        assert oracle.layernorm_sums(row) == (_to_f64(s1), _to_f64(d))


def test_layernorm_sums_large_mean_small_spread():
    # 2^20 everywhere but one 2^20 + 2^13: a one-pass fp32 E[x^2] - E[x]^2 loses this
    # variance entirely; here S1 = K 2^20 + 2^13 and D = (K - 1) 2^26 exactly
    for K in (8, 100, 4096):
        row = np.full(K, 2.0 ** 20, np.float32)
        row[K // 3] += 2.0 ** 13
        s1, d = oracle.layernorm_sums(_bf(row))
        assert s1 == K * 2.0 ** 20 + 2.0 ** 13
        assert d == (K - 1) * 2.0 ** 26
    # the bf16 extremes: the smallest subnormal and the largest finite value
    s1, d = oracle.layernorm_sums(np.array([0x0001, 0x0000], np.uint16))
    assert s1 == 2.0 ** -133 and d == 2.0 ** -266
    s1, d = oracle.layernorm_sums(np.array([0x7F7F, 0xFF7F], np.uint16))
    assert s1 == 0.0 and d == 2 * 2 * (255.0 * 2.0 ** 120) ** 2


def test_layernorm_h_from_the_exact_sums():
    # mean = fp64(S1) / K, var = fp64(D) / K^2, r = 1 / sqrt(var + eps),
    # h = bf16(fl32((x' - mean) r)), recomputed from the exact rational sums
    rng = np.random.default_rng(25)
    X = np.concatenate([_wide_bf16_rows(rng, 3, 96) & np.uint16(0xBFFF),
                        _bf((2.0 + 0.3 * rng.standard_normal((3, 96))).astype(np.float32))])
    eps = np.float32(1e-5)
    _, h = oracle.layernorm(X, eps=float(eps))
    for i in range(X.shape[0]):
        s1, d = _exact_moments(X[i])
        mean = _to_f64(s1) / 96
        r = 1.0 / math.sqrt(_to_f64(d) / (96.0 * 96.0) + float(eps))
        dev = (_f(X[i]).astype(np.float64) - mean) * r
        assert np.array_equal(h[i], _bf(dev.astype(np.float32))), i


def test_layernorm_matches_the_library_layer_norm():
    # torch's non-affine layer_norm (the listing's F.layer_norm) in fp64 on x', rounded
    # the same way: at most one bf16 ulp apart (a different rounding of mean and
    # variance), and nearly always identical
    rng = np.random.default_rng(26)
    X = _bf((0.7 + 2.0 * rng.standard_normal((16, 2560))).astype(np.float32))
    _, h = oracle.layernorm(X)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(_f(X).astype(np.float64)), [2560],
                                         eps=float(np.float32(1e-5)))
    ref_bits = _bf(ref.numpy().astype(np.float32)).astype(np.int32)
    diff = np.abs(h.astype(np.int32) - ref_bits)
    assert diff.max() <= 1
    assert np.mean(diff == 0) > 0.99


def test_layernorm_output_moments():
    rng = np.random.default_rng(27)
    X = _bf((-4.0 + 3.0 * rng.standard_normal((8, 2560))).astype(np.float32))
    _, h = oracle.layernorm(X)
    hf = _f(h).astype(np.float64)
    # each h within half a bf16 ulp (2^-9 relative) of the exact standardized value
    assert np.all(np.abs(hf.mean(axis=1)) < 2.0 ** -8)
    assert np.all(np.abs((hf ** 2).mean(axis=1) - 1.0) < 2 * 2.0 ** -8)


def test_layernorm_residual_add_as_rmsnorm():
    rng = np.random.default_rng(28)
    X = _bf(rng.standard_normal((3, 64)).astype(np.float32))
    D = _bf(rng.standard_normal((3, 64)).astype(np.float32))
    x1, _ = oracle.layernorm(X, D)
    x2, _ = oracle.rmsnorm(X, D)
    assert np.array_equal(x1, x2)
    a = oracle.layernorm(X)
    b = oracle.layernorm(X, np.zeros_like(X))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- Hadamard rotation
# ("BitNet a4.8 Guide", "Best Practices for Deploying BitNet a4.8 in Production",
# Outlier Suppression row; readings in tests/golden/hadamard_examples.json)

def _hadamard_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "hadamard_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("K,b", [(4, 4), (12, 4), (48, 16), (256, 256), (2560, 512),
                                 (6912, 256), (8192, 8192), (16384, 8192), (24576, 8192)])
def test_hadamard_block_sizes(K, b):
    # the largest power of two dividing K, at most 8192
    assert oracle.hadamard_block(K) == b


def test_hadamard_worked_examples():
    for ex in _hadamard_golden()["rows"]:
        x = np.array([ex["x"]], np.float32)
        assert oracle.hadamard_block(ex["K"]) == ex["b"]
        np.testing.assert_array_equal(oracle.hadamard_rows(x)[0], np.array(ex["y"], np.float32),
                                      err_msg=ex["name"])


def test_hadamard_unit_vectors_are_hadamard_rows():
    # x = e_j -> row j of the Sylvester matrix: (-1)^popcount(i & j), scipy's construction
    from scipy.linalg import hadamard
    b = 64
    H = hadamard(b)
    X = np.eye(b, dtype=np.float32)
    Y = oracle.hadamard_rows(X)
    np.testing.assert_array_equal(Y, H.astype(np.float32))
    pop = np.array([[bin(i & j).count("1") for i in range(b)] for j in range(b)])
    np.testing.assert_array_equal(Y, ((-1.0) ** pop).astype(np.float32))


@pytest.mark.parametrize("K,dtype", [(1536, "f32"), (2560, "bf16"), (8192, "f32")])
def test_hadamard_matches_dense_product(K, dtype):
    # against X @ blockdiag(H_b) in float64: the fp32 fast transform is within its
    # rounding bound log2(b) * 2^-24 * sum |x| (over the block) of every output
    from scipy.linalg import hadamard
    rng = np.random.default_rng(5)
    X = rng.standard_normal((3, K)).astype(np.float32)
    X[:, 7] *= 40.0  # an outlier channel
    Xin = workloads.to_bf16_bits(X) if dtype == "bf16" else X
    Xf = workloads.bf16_bits_to_f32(Xin) if dtype == "bf16" else X
    b = oracle.hadamard_block(K)
    H = hadamard(b).astype(np.float64)
    Y = oracle.hadamard_rows(Xin).astype(np.float64)
    L = int(math.log2(b))
    for j0 in range(0, K, b):
        blk = Xf[:, j0:j0 + b].astype(np.float64)
        ref = blk @ H
        bound = L * 2.0 ** -24 * np.abs(blk).sum(axis=1, keepdims=True) * 1.0001
        assert (np.abs(Y[:, j0:j0 + b] - ref) <= bound).all()


def test_hadamard_involution_exact():
    # small integers keep every intermediate exact in fp32: H (H x) = b x
    rng = np.random.default_rng(6)
    X = rng.integers(-64, 65, (4, 512)).astype(np.float32)
    b = oracle.hadamard_block(512)
    np.testing.assert_array_equal(oracle.hadamard_rows(oracle.hadamard_rows(X)), b * X)


def test_rotation_folds_into_both_operands_exactly():
    # (X H)(W H)^T / b = X W^T, exactly for small integers (no quantization involved)
    rng = np.random.default_rng(7)
    K = 48
    X = rng.integers(-8, 9, (3, K)).astype(np.float32)
    W = rng.integers(-3, 4, (5, K)).astype(np.float32)
    b = oracle.hadamard_block(K)
    lhs = oracle.hadamard_rows(X).astype(np.float64) @ oracle.hadamard_rows(W).astype(np.float64).T / b
    np.testing.assert_array_equal(lhs, X.astype(np.float64) @ W.astype(np.float64).T)


def test_rotated_weights_worked_example():
    ex = _hadamard_golden()["weights"]
    W = np.array(ex["W"], np.float32)
    packed, g, codes = oracle.quantize_weights_rotated(W)
    np.testing.assert_array_equal(codes, np.array(ex["codes"], np.int8))
    np.testing.assert_array_equal(packed[:, 0], np.array(ex["packed"], np.uint8))
    assert g == np.float32(ex["gamma"])


def test_rotated_acts_worked_example():
    ex = _hadamard_golden()["acts_int4"]
    X = np.array([ex["x"]], np.float32)
    xq, s = oracle.quantize_acts_rotated(X, bits=4)
    np.testing.assert_array_equal(xq[0], np.array(ex["bytes"], np.uint8))
    np.testing.assert_array_equal(_unpack_nibbles(xq, 4)[0], np.array(ex["codes"]))
    assert f32_bits(s[0]) == _bits(ex["scale_bits"])


@pytest.mark.parametrize("K", [256, 2560])
def test_rotated_gamma_is_rotated_mean_over_b(K):
    # gamma = (exact mean |W H|, rounded once) / b, and the codes are those of W H
    rng = np.random.default_rng(8)
    W = (0.02 * rng.standard_normal((64, K))).astype(np.float32)
    b = oracle.hadamard_block(K)
    R = oracle.hadamard_rows(W)
    packed, g, codes = oracle.quantize_weights_rotated(W)
    ref = Fraction(sum(frac_of_f32(abs(float(v))) for v in R.ravel()), R.size)
    assert f32_bits(g * np.float32(b)) == f32_bits(round_to_f32(ref))
    p2, g2, c2 = oracle.quantize_weights(R)
    np.testing.assert_array_equal(codes, c2)
    assert g * np.float32(b) == g2


def test_rotation_spreads_an_outlier():
    # one channel 100x the others: rotated, its energy is spread over the block, so the
    # absmax falls towards the rms (the point of the rotation before 4-bit codes)
    rng = np.random.default_rng(9)
    X = rng.standard_normal((8, 512)).astype(np.float32)
    X[:, 3] = 100.0
    R = oracle.hadamard_rows(X)
    ratio = lambda A: (np.abs(A).max(axis=1) / np.sqrt((A.astype(np.float64) ** 2).mean(axis=1)))
    assert (ratio(X) > 15).all() and (ratio(R) < 5).all()


# ---------------------------------------------------------------- backward (STE)
# int8: "BitNet b1.58 ...", "Implementation" Step 1-2 listings; int4: "BitNet a4.8
# Guide", "Implementation" Step 2-3 listings.  The pin: float64 autograd through each
# listing's own forward, with straight-through functions carrying the listing's masks,
# so that the chain rule (which operand, which transpose, where the scales go) comes
# from the library, not from the oracle's formulas.

def _bwd_case(M, N, K, bits, gran=oracle.PER_TOKEN, seed=0, bias=True):
    rng = np.random.default_rng([seed, M, N, K, bits])
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[0, 0] = 2.0   # masked by the int4 weight STE (|w| > 1.5)
    W[0, 1] = -1.5  # not masked (the test is strict)
    X = rng.standard_normal((M, K)).astype(np.float32)
    packed, g, codes = oracle.quantize_weights(W)
    xq, s = oracle.quantize_acts(X, bits=bits, gran=gran)
    dY = workloads.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    return W, X, packed, g, codes, xq, s, dY


def _autograd_ref(W, X, codes, g, xq, s, dY, bits, gran, K):
    torch64 = torch.float64
    q = (xq.astype(np.int64) if bits == 8 else _unpack_nibbles(xq, K)).astype(np.float64)
    c = codes.astype(np.float64)
    sv = np.asarray(s, np.float32)
    srow = sv if gran == oracle.PER_TOKEN else np.full(X.shape[0], sv[0], np.float32)
    x = torch.tensor(X.astype(np.float64), requires_grad=True)
    w = torch.tensor(W.astype(np.float64), requires_grad=True)
    bias = torch.zeros(W.shape[0], dtype=torch64, requires_grad=True)
    dy = torch.tensor(workloads.bf16_bits_to_f32(dY).astype(np.float64))

    class Pass(torch.autograd.Function):  # forward: the given value; backward: identity
        @staticmethod
        def forward(ctx, inp, val):
            return val

        @staticmethod
        def backward(ctx, grad):
            return grad, None

    class MaskedAct(torch.autograd.Function):  # [a48] ActivationA4Quantizer
        @staticmethod
        def forward(ctx, inp, val, scale32):
            ctx.save_for_backward(inp, scale32)
            return val

        @staticmethod
        def backward(ctx, grad):
            inp, scale32 = ctx.saved_tensors
            norm = torch.from_numpy((inp.detach().numpy().astype(np.float32) /
                                     scale32.numpy()[:, None]).astype(np.float32))
            grad = grad.clone()
            grad[(norm < -8.0) | (norm > 7.0)] = 0.0
            return grad, None, None

    class MaskedW(torch.autograd.Function):  # [a48] WeightTernaryQuantizer
        @staticmethod
        def forward(ctx, inp, val):
            ctx.save_for_backward(inp)
            return val

        @staticmethod
        def backward(ctx, grad):
            (inp,) = ctx.saved_tensors
            grad = grad.clone()
            grad[inp.abs() > 1.5] = 0.0
            return grad, None

    if bits == 8:  # y = linear(q, c) * (gamma / s) + bias, f in fp32 as the listing has it
        f = (np.float32(g) / srow).astype(np.float32).astype(np.float64)
        y = torch.nn.functional.linear(Pass.apply(x, torch.tensor(q)), Pass.apply(w, torch.tensor(c)))
        y = y * torch.tensor(f)[:, None] + bias
    else:  # y = linear(q s, c gamma) + bias, the dequantized operands in fp32
        xdq = (q.astype(np.float32) * srow[:, None]).astype(np.float32).astype(np.float64)
        wdq = (c.astype(np.float32) * np.float32(g)).astype(np.float64)
        y = torch.nn.functional.linear(MaskedAct.apply(x, torch.tensor(xdq), torch.tensor(srow)),
                                       MaskedW.apply(w, torch.tensor(wdq))) + bias
    (y * dy).sum().backward()
    return x.grad.numpy(), w.grad.numpy(), bias.grad.numpy()


@pytest.mark.parametrize("bits,gran", [(8, oracle.PER_TOKEN), (4, oracle.PER_TOKEN),
                                       (8, oracle.PER_TENSOR), (4, oracle.PER_TENSOR)])
def test_backward_matches_autograd(bits, gran):
    M, N, K = 6, 40, 64
    W, X, packed, g, codes, xq, s, dY = _bwd_case(M, N, K, bits, gran)
    got = oracle.backward(dY, xq, bits, s, gran, packed, g, X=X, W=W)
    rx, rw, rb = _autograd_ref(W, X, codes, g, xq, s, dY, bits, gran, K)
    # the oracle rounds dz = dY * f to fp32 (int8), as the listing's fp32 graph does;
    # autograd in float64 does not: within 2^-23 of the sum of |terms|
    dyf = workloads.bf16_bits_to_f32(dY).astype(np.float64)
    tx = 2.0 ** -23 * (np.abs(dyf) @ np.abs(codes.astype(np.float64))) * (10.0 if bits == 8 else g)
    np.testing.assert_allclose(got["dX"], rx, rtol=0, atol=float(tx.max()) + 1e-300)
    q = (xq.astype(np.int64) if bits == 8 else _unpack_nibbles(xq, K)).astype(np.float64)
    srow = np.broadcast_to(np.asarray(s, np.float64), (M,)) if len(s) == 1 else s.astype(np.float64)
    fm = (np.float64(g) / srow) if bits == 8 else srow  # per-token factor of the dW terms
    tw = 2.0 ** -23 * ((np.abs(dyf) * fm[:, None]).T @ np.abs(q)) * 1.01
    np.testing.assert_allclose(got["dW"], rw, rtol=0, atol=float(tw.max()) + 1e-300)
    assert (np.abs(got["dW"] - rw) <= tw + 1e-300).all()
    np.testing.assert_array_equal(got["dbias"], rb)
    if bits == 4:  # the listing's weight mask: |w| = 2 masked, |w| = 1.5 not
        assert got["dW"][0, 0] == 0.0 and got["dW"][0, 1] != 0.0


def test_backward_one_hot_closed_form():
    M, N, K = 4, 8, 32
    for bits in (8, 4):
        W, X, packed, g, codes, xq, s, _ = _bwd_case(M, N, K, bits, seed=3)
        m0, n0 = 2, 5
        dY = np.zeros((M, N), np.uint16)
        dY[m0, n0] = workloads.to_bf16_bits(np.array([[1.5]], np.float32))[0, 0]
        got = oracle.backward(dY, xq, bits, s, oracle.PER_TOKEN, packed, g)
        q = (xq.astype(np.int64) if bits == 8 else _unpack_nibbles(xq, K)).astype(np.float64)
        if bits == 8:
            dz = np.float64(np.float32(1.5) * (np.float32(g) / s[m0]))
            ex_dx, ex_dw = dz * codes[n0], dz * q[m0]
        else:
            ex_dx = 1.5 * codes[n0] * np.float64(g)
            ex_dw = 1.5 * (q[m0].astype(np.float32) * s[m0]).astype(np.float64)
        assert (got["dX"][np.arange(M) != m0] == 0).all() and (got["dW"][np.arange(N) != n0] == 0).all()
        np.testing.assert_array_equal(got["dX"][m0], ex_dx)
        np.testing.assert_array_equal(got["dW"][n0], ex_dw)


def test_backward_int4_activation_mask_edge():
    # x / s rounds to 7.0000005 for the token's own maximum: the listing zeroes it
    K = 32
    X = np.zeros((1, K), np.float32)
    X[0, 3] = np.float32(9.360724449157715)
    X[0, 4] = np.float32(1.0)
    xq, s = oracle.quantize_acts(X, bits=4)
    assert np.float32(X[0, 3]) / s[0] > np.float32(7.0)
    W = (0.02 * np.random.default_rng(1).standard_normal((4, K))).astype(np.float32)
    packed, g, _ = oracle.quantize_weights(W)
    dY = workloads.to_bf16_bits(np.ones((1, 4), np.float32))
    got = oracle.backward(dY, xq, 4, s, oracle.PER_TOKEN, packed, g, X=X)
    free = oracle.backward(dY, xq, 4, s, oracle.PER_TOKEN, packed, g)
    assert got["dX"][0, 3] == 0.0 and free["dX"][0, 3] != 0.0
    np.testing.assert_array_equal(np.delete(got["dX"][0], 3), np.delete(free["dX"][0], 3))


def test_backward_is_linear_in_dy():
    M, N, K = 5, 12, 48
    W, X, packed, g, codes, xq, s, dY1 = _bwd_case(M, N, K, 4, seed=4)
    dY2 = workloads.to_bf16_bits(np.random.default_rng(5).integers(-4, 5, (M, N)).astype(np.float32))
    dY1 = workloads.to_bf16_bits(np.random.default_rng(6).integers(-4, 5, (M, N)).astype(np.float32))
    dYs = workloads.to_bf16_bits(workloads.bf16_bits_to_f32(dY1) + workloads.bf16_bits_to_f32(dY2))
    a = oracle.backward(dY1, xq, 4, s, 0, packed, g, X=X, W=W)
    b = oracle.backward(dY2, xq, 4, s, 0, packed, g, X=X, W=W)
    c = oracle.backward(dYs, xq, 4, s, 0, packed, g, X=X, W=W)
    for k in ("dX", "dW", "dbias"):
        np.testing.assert_allclose(c[k], a[k] + b[k], rtol=1e-12, atol=1e-12)
