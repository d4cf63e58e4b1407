"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by
element, on the same seeded inputs.

Bar: packed weights, gamma, activation codes, scales and int32 accumulators
bit-identical; outputs within 1e-5 relative in fp32 / one ulp in bf16 and, since
both sides fix the same fp32 operation order, bit-identical too.
Small shapes are compared in full; the full-size shapes (2B decode/prefill, 70B
layer) on sampled outputs the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import (assert_same_bytes, assert_y_matches, bits32, sample_positions, say,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu

YD = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16),
      "i32": (torch.int32, None)}


def _weights_case(kind, n, k, seed=0):
    rng = np.random.default_rng([seed, n, k])
    if kind == "gauss":
        return (np.float32(0.02) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    if kind == "ternary":
        return workloads.ternary_weights(rng, n, k)
    if kind == "zeros":
        return np.zeros((n, k), np.float32)
    if kind == "tiny":  # mean far below eps -> gamma = eps, codes mostly 0
        return (1e-9 * rng.standard_normal((n, k))).astype(np.float32)
    if kind == "halfgrid":  # many exact ties at gamma/2 multiples
        return (rng.integers(-4, 5, (n, k)) * 0.25).astype(np.float32)
    if kind == "wide":  # exponents over the whole finite range, subnormals included
        mag = np.ldexp(1.0 + rng.random((n, k)), rng.integers(-150, 120, (n, k)))
        return (np.where(rng.random((n, k)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    raise ValueError(kind)


# ---------------------------------------------------------------- weights

@pytest.mark.parametrize("kind,n,k,dtype", [
    ("gauss", 512, 256, "f32"),
    ("gauss", 512, 256, "bf16"),
    ("gauss", 1, 16, "f32"),
    ("gauss", 3, 48, "f32"),
    ("gauss", 37, 80, "bf16"),
    ("zeros", 16, 64, "f32"),
    ("tiny", 33, 32, "f32"),
    ("halfgrid", 64, 128, "f32"),
    ("wide", 300, 512, "f32"),
    ("wide", 1000, 1024, "bf16"),
    ("ternary", 6912, 2560, "f32"),
    ("ternary", 2560, 6912, "f32"),
    ("gauss", 7680, 2560, "bf16"),
    ("gauss", 2560, 6912, "f32"),
])
def test_quantize_weights_parity(kind, n, k, dtype):
    W = _weights_case(kind, n, k)
    Win = workloads.to_bf16_bits(W) if dtype == "bf16" else W
    say("quantize_weights", kind, n, k, dtype)
    packed, gamma = bl.quantize_weights(to_dev(Win))
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights(Win)
    assert bits32(to_host(gamma))[0] == bits32(np.array([g_ref]))[0], "gamma differs"
    assert_same_bytes(to_host(packed), p_ref, "packed weights")


def test_quantize_weights_70b_layer():
    codes, _ = workloads.layer_70b(m=1)
    W = codes.astype(np.float32)
    say("quantize_weights 70B layer", W.shape)
    packed, gamma = bl.quantize_weights(to_dev(W))
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    assert bits32(to_host(gamma))[0] == bits32(np.array([g_ref]))[0]
    assert_same_bytes(to_host(packed), p_ref, "packed weights 28672x8192")


# ---------------------------------------------------------------- activations

def _acts_case(m, k, seed=0, outliers=4, factor=20.0, zero_row=False):
    X = workloads.outlier_acts(np.random.default_rng([seed, m, k]), m, k, outliers if k > 64 else 0,
                               factor)
    if zero_row and m > 1:
        X[1] = 0.0
    return X


@pytest.mark.parametrize("m,k", [(8, 256), (1, 2560), (1, 6912), (3, 16), (5, 48), (7, 8192),
                                 (2048, 2560), (2048, 6912)])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_acts_parity(m, k, bits, gran, dtype):
    X = _acts_case(m, k, zero_row=True)
    Xin = workloads.to_bf16_bits(X) if dtype == "bf16" else X
    say("quantize_acts", m, k, bits, gran, dtype)
    xq, s = bl.quantize_acts(to_dev(Xin), bits=bits, gran=gran)
    torch.cuda.synchronize()
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts(Xin, bits=bits, gran=g)
    assert_same_bytes(bits32(to_host(s)), bits32(s_ref), "act_scale")
    assert_same_bytes(to_host(xq), xq_ref, "activation codes")


def test_quantize_acts_70b_layer_outliers():
    _, X = workloads.layer_70b()
    for bits in (8, 4):
        say("quantize_acts 70B layer", X.shape, bits)
        xq, s = bl.quantize_acts(to_dev(X), bits=bits)
        torch.cuda.synchronize()
        xq_ref, s_ref = oracle.quantize_acts(X, bits=bits)
        assert_same_bytes(bits32(to_host(s)), bits32(s_ref), "act_scale")
        assert_same_bytes(to_host(xq), xq_ref, "activation codes")


# ---------------------------------------------------------------- forward

def _layer(m, k, n, seed, kind="gauss"):
    W = _weights_case(kind, n, k, seed)
    X = _acts_case(m, k, seed=seed)
    return W, X


def _run_forward(W, X, bits, gran, epi, ydt, bias, fused, x_dtype="f32"):
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    Xin = workloads.to_bf16_bits(X) if x_dtype == "bf16" else X
    Wd = to_dev(W)
    packed, gamma = bl.quantize_weights(Wd)
    bias_d = to_dev(bias) if bias is not None else None
    tdt, _ = YD[ydt]
    if fused:
        y = bl.forward_fused(to_dev(Xin), packed, gamma, bits=bits, gran=gran, bias=bias_d,
                             epilogue=epi, out_dtype=tdt)
    else:
        xq, s = bl.quantize_acts(to_dev(Xin), bits=bits, gran=gran)
        y = bl.forward(xq, s, packed, gamma, bits=bits, gran=gran, bias=bias_d, epilogue=epi,
                       out_dtype=tdt)
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    xq_ref, s_ref = oracle.quantize_acts(Xin, bits=bits, gran=g)
    return to_host(y), (p_ref, g_ref, xq_ref, s_ref, g)


def _check_forward(M, K, N, bits, gran, epi, ydt, with_bias, fused, x_dtype="f32", seed=0,
                   kind="gauss", sampled=None):
    W, X = _layer(M, K, N, seed, kind)
    bias = (np.random.default_rng(seed).standard_normal(N).astype(np.float32)
            if with_bias else None)
    say("forward", dict(M=M, K=K, N=N, bits=bits, gran=gran, epi=epi, y=ydt, bias=with_bias,
                        fused=fused, x=x_dtype))
    y, (p_ref, g_ref, xq_ref, s_ref, g) = _run_forward(W, X, bits, gran, epi, ydt, bias, fused,
                                                       x_dtype)
    e = oracle.EPI_RELU2 if epi == "relu2" else oracle.EPI_NONE
    _, odt = YD[ydt]
    if sampled is None:
        sampled = M * N * K > 3e8
    if not sampled:
        y_ref, acc_ref = oracle.forward(xq_ref, bits, s_ref, g, p_ref, g_ref, bias=bias, epi=e,
                                        y_dtype=odt if odt is not None else oracle.F32)
        ref = acc_ref if ydt == "i32" else y_ref
        assert_y_matches(y, ref, ydt, "Y")
    else:
        ms, ns = sample_positions(M, N, 4096, seed)
        y_ref, acc_ref = oracle.forward_at(xq_ref, bits, s_ref, g, p_ref, g_ref, ms, ns,
                                           bias=bias, epi=e,
                                           y_dtype=odt if odt is not None else oracle.F32)
        ref = acc_ref if ydt == "i32" else y_ref
        assert_y_matches(y[ms, ns], ref, ydt, "Y (sampled)")


# decode path (GEMV, M <= 8, K % 64 == 0)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 11, 16])
@pytest.mark.parametrize("K,N", [(256, 512), (64, 17), (2560, 300), (6912, 129)])
@pytest.mark.parametrize("bits", [8, 4])
def test_forward_decode_shapes(M, K, N, bits):
    _check_forward(M, K, N, bits, "token", None, "i32", False, False)
    _check_forward(M, K, N, bits, "token", "relu2", "f32", True, False)


@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("epi", [None, "relu2"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("fused", [False, True])
def test_forward_decode_variants(gran, epi, ydt, fused):
    for bits in (8, 4):
        _check_forward(4, 256, 512, bits, gran, epi, ydt, False, fused)
        _check_forward(1, 2560, 6912, bits, gran, epi, ydt, False, fused, x_dtype="bf16",
                       kind="ternary")


# fused forward of 5..16 bf16 tokens (the quantizer's own launch, then the GEMV on the
# codes); bf16 inputs put many quotients exactly on rounding ties (x = a/2), which the
# codes must break as defined
@pytest.mark.parametrize("M", [5, 8, 11, 16])
@pytest.mark.parametrize("K,N", [(256, 512), (2560, 2560), (640, 300), (1024, 4096)])
@pytest.mark.parametrize("bits", [8, 4])
def test_forward_fused_mid_m(M, K, N, bits):
    _check_forward(M, K, N, bits, "token", "relu2", "f32", True, True, x_dtype="bf16")
    _check_forward(M, K, N, bits, "tensor", None, "i32", False, True, x_dtype="bf16")
    _check_forward(M, K, N, bits, "token", None, "bf16", False, True, x_dtype="bf16", kind="ternary")


# prefill path (MFMA GEMM)
@pytest.mark.parametrize("M,K,N", [(9, 256, 512), (130, 48, 37), (200, 336, 300),
                                   (128, 128, 128), (257, 2560, 129), (64, 6912, 200)])
@pytest.mark.parametrize("bits", [8, 4])
def test_forward_prefill_shapes(M, K, N, bits):
    _check_forward(M, K, N, bits, "token", None, "i32", False, False)
    _check_forward(M, K, N, bits, "tensor", "relu2", "f32", True, False)


@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("epi", [None, "relu2"])
@pytest.mark.parametrize("ydt", ["f32", "bf16", "i32"])
def test_forward_prefill_variants(gran, epi, ydt):
    if ydt == "i32" and epi:
        pytest.skip("raw accumulators take no epilogue")
    for bits in (8, 4):
        _check_forward(300, 512, 260, bits, gran, epi, ydt, ydt != "i32", bits == 4)


# few large tiles and a long K (the 128-wide tile path with one 4-wave block per tile):
# both entry points, every output type, ragged last row / column tiles
@pytest.mark.parametrize("M,K,N", [(300, 4096, 300), (512, 3072, 1000), (128, 3072, 128),
                                   (1000, 6400, 520)])
@pytest.mark.parametrize("ydt", ["f32", "bf16", "i32"])
def test_forward_prefill_long_k(M, K, N, ydt):
    _check_forward(M, K, N, 8, "token", None if ydt == "i32" else "relu2", ydt, ydt != "i32", False)
    _check_forward(M, K, N, 8, "tensor", None, ydt, False, True, x_dtype="bf16")


# rows longer than the activation preparation keeps in registers (8192 elements per
# 256-thread row): the groups past them are read a second time, and the reorder of
# quantized codes takes two rounds of eight loads per lane
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("gran", ["token", "tensor"])
def test_forward_prefill_rows_past_registers(xdt, gran):
    for fused in (False, True):
        _check_forward(260, 12288, 136, 8, gran, "relu2", "f32", True, fused, x_dtype=xdt,
                       sampled=False)


# 4-bit activations from raw rows at prefill sizes (int4 codes, their FP6 operand blocks,
# the FP6 x FP4 GEMM).  Ragged token counts (padding inside the last 32-token group and
# up to the 256-token multiple), both input types, per-tensor scales, and K = 8256 (129 k
# blocks: the last of the 16 code-sum ranges is empty); raw int32 accumulators and
# rescaled outputs in full
@pytest.mark.parametrize("M,K,N,xdt,gran", [(130, 512, 136, "bf16", "token"),
                                            (257, 2560, 129, "f32", "token"),
                                            (300, 8256, 200, "f32", "tensor"),
                                            (137, 8256, 160, "bf16", "token"),
                                            (512, 1024, 384, "bf16", "tensor")])
def test_forward_fused_int4_fp6_blocks(M, K, N, xdt, gran):
    _check_forward(M, K, N, 4, gran, None, "i32", False, True, x_dtype=xdt, sampled=False)
    _check_forward(M, K, N, 4, gran, "relu2", "f32", True, True, x_dtype=xdt, sampled=False)


def _codes_f64(xq_ref, bits, p_ref, K):
    """The oracle's activation and weight codes as float64 matrices, unpacked from the
    documented layouts (int4: element 2i in the low nibble; 2-bit field c + 1 of code k in
    bits 2 (k % 4) of byte k / 4)."""
    if bits == 8:
        q = xq_ref.astype(np.float64)
    else:
        lo = (xq_ref & 0xF).astype(np.int16)
        hi = (xq_ref >> 4).astype(np.int16)
        v = np.stack([lo, hi], axis=-1).reshape(xq_ref.shape[0], K)
        q = np.where(v >= 8, v - 16, v).astype(np.float64)
    f = np.stack([(p_ref >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(p_ref.shape[0], K)
    return q, f.astype(np.float64) - 1.0


# full-size 2B shapes: outputs sampled; the int32 accumulators in full, against a float64
# matmul of the oracle's codes (exact: every partial sum is an integer below 2^53)
@pytest.mark.parametrize("shape,epi", [(workloads.SHAPE_UP, "relu2"), (workloads.SHAPE_DOWN, None)])
@pytest.mark.parametrize("bits", [8, 4])
def test_forward_prefill_2b_shapes(shape, epi, bits):
    K, N = shape
    _check_forward(2048, K, N, bits, "token", epi, "bf16", False, True, x_dtype="bf16",
                   kind="ternary", sampled=True)
    W, X = _layer(2048, K, N, 0, "ternary")
    say("forward 2B prefill, full int32 accumulators", K, N, bits)
    acc, (p_ref, _, xq_ref, _, _) = _run_forward(W, X, bits, "token", None, "i32", None, False,
                                                 "bf16")
    q, c = _codes_f64(xq_ref, bits, p_ref, K)
    assert np.array_equal(acc.astype(np.float64), q @ c.T), "int32 accumulators differ"


@pytest.mark.parametrize("shape,epi", [(workloads.SHAPE_UP, "relu2"), (workloads.SHAPE_DOWN, None)])
def test_forward_decode_2b_shapes_full(shape, epi):
    K, N = shape
    for bits in (8, 4):
        _check_forward(1, K, N, bits, "token", epi, "bf16", False, True, x_dtype="bf16",
                       kind="ternary", sampled=False)
        _check_forward(1, K, N, bits, "token", None, "i32", False, True, x_dtype="bf16",
                       kind="ternary", sampled=False)


def test_forward_70b_layer_sampled():
    codes, X = workloads.layer_70b()
    W = codes.astype(np.float32)
    del codes
    Wd = to_dev(W)
    packed, gamma = bl.quantize_weights(Wd)
    del Wd
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    del W
    Xd = to_dev(X)
    M, K = X.shape
    N = packed.shape[0]
    ms, ns = sample_positions(M, N, 4096, 4)
    for bits in (8, 4):
        say("forward 70B layer", bits)
        y = bl.forward_fused(Xd, packed, gamma, bits=bits, out_dtype=torch.bfloat16)
        acc_w = bl.quantize_acts(Xd, bits=bits)
        acc = bl.forward(acc_w[0], acc_w[1], packed, gamma, bits=bits, out_dtype=torch.int32)
        torch.cuda.synchronize()
        xq_ref, s_ref = oracle.quantize_acts(X, bits=bits)
        y_ref, acc_ref = oracle.forward_at(xq_ref, bits, s_ref, 0, p_ref, g_ref, ms, ns,
                                           y_dtype=oracle.BF16)
        yh = to_host(y)
        assert_y_matches(yh[ms, ns], y_ref, "bf16", "Y 70B layer")
        assert_same_bytes(to_host(acc)[ms, ns], acc_ref, "acc 70B layer")
        del y, acc


def test_forward_edge_zero_weights_and_rows():
    M, K, N = 5, 128, 64
    W = np.zeros((N, K), np.float32)
    X = _acts_case(M, K)
    X[2] = 0.0
    for fused in (False, True):
        y, _ = _run_forward(W, X, 8, "token", "relu2", "f32", None, fused)
        assert (y == 0).all()
    W = _weights_case("gauss", N, K)
    y, _ = _run_forward(W, X, 8, "token", None, "f32", None, False)
    assert (y[2] == 0).all()


def test_forward_deterministic():
    W, X = _layer(2048, 2560, 600, 3, "ternary")
    Xd, Wd = to_dev(X), to_dev(W)
    packed, gamma = bl.quantize_weights(Wd)
    outs = []
    for _ in range(2):
        xq, s = bl.quantize_acts(Xd)
        outs.append(to_host(bl.forward(xq, s, packed, gamma, out_dtype=torch.int32)))
    assert_same_bytes(outs[0], outs[1], "repeat run")
    p2, g2 = bl.quantize_weights(Wd)
    assert_same_bytes(to_host(p2), to_host(packed), "repeat pack")


def _near_tie_acts(m, k, bits, seed=0):
    """fp32 rows whose codes sit on rounding decisions: each row's absmax a is pinned at
    column 0, and the other columns hold t = fl(h * s) for every half-integer h that
    |x| <= a allows (s = fl(a / 7) for 4 bits, x = h / s8 with s8 = fl(127 / a) for 8
    bits), and t's neighbours up to 3 ulps either side.  Scales with short mantissas
    make some of these exact ties (round half to even decides)."""
    rng = np.random.default_rng([seed, m, k, bits])
    X = np.zeros((m, k), dtype=np.float32)
    amaxes = [5.25, 1.0, 3.3, 0.0173, 1.0e4, 7.0, 0.4375, 123.456]
    for r in range(m):
        a = np.float32(amaxes[r % len(amaxes)] * (1.0 if r < len(amaxes) else rng.uniform(0.5, 2)))
        vals = []
        if bits == 4:
            sc = np.float32(a) / np.float32(7.0)
            hs = [h + 0.5 for h in range(-7, 7)]
            base = [np.float32(np.float32(h) * sc) for h in hs]
        else:
            s8 = np.float32(127.0) / np.float32(a)
            hs = [h + 0.5 for h in range(-127, 127, 7)]
            base = [np.float32(np.float32(h) / s8) for h in hs]
        for t in base:
            v = t
            for _ in range(3):
                v = np.nextafter(v, np.float32(np.inf), dtype=np.float32)
                vals.append(v)
            v = t
            for _ in range(3):
                v = np.nextafter(v, np.float32(-np.inf), dtype=np.float32)
                vals.append(v)
            vals.append(t)
        vals = [v for v in vals if abs(v) <= a]
        rng.shuffle(vals)
        n = min(len(vals), k - 1)
        X[r, 0] = a if r % 2 == 0 else -a
        X[r, 1:1 + n] = vals[:n]
    return X


# activation codes on rounding decisions: x / s (4 bits) or x * s (8 bits) at, and a
# few ulps around, every half-integer, against the oracle's exact quotient and product;
# through the quantizer, the fused GEMV prologue (M <= 4) and the streaming kernel's
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("gran", ["token", "tensor"])
def test_quantize_acts_near_ties(bits, gran):
    say("quantize_acts near ties", bits, gran)
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    X = _near_tie_acts(16, 256, bits)
    xq, s = bl.quantize_acts(to_dev(X), bits=bits, gran=gran)
    torch.cuda.synchronize()
    xq_ref, s_ref = oracle.quantize_acts(X, bits=bits, gran=g)
    assert_same_bytes(bits32(to_host(s)), bits32(s_ref), "act_scale")
    assert_same_bytes(to_host(xq), xq_ref, "activation codes")
    # fused forward, M <= 4: quantization in the GEMV prologue; int32 accumulators
    W = _weights_case("gauss", 64, 256, seed=3)
    packed, gamma = bl.quantize_weights(to_dev(W))
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    for m0 in (0, 4, 8):
        Xm = np.ascontiguousarray(X[m0:m0 + 4])
        y = bl.forward_fused(to_dev(Xm), packed, gamma, bits=bits, gran=gran, out_dtype=torch.int32)
        torch.cuda.synchronize()
        xq_m, s_m = oracle.quantize_acts(Xm, bits=bits, gran=g)
        _, acc_ref = oracle.forward(xq_m, bits, s_m, g, p_ref, g_ref, y_dtype=oracle.F32)
        assert_same_bytes(to_host(y), acc_ref, "fused accumulators rows %d.." % m0)
    # streaming kernel (64 problems x 2048 rows): its prologue quantizes too
    B, N = 64, 2048
    Xb = np.stack([X[(4 * b) % 16:(4 * b) % 16 + 4] for b in range(B)])
    Wb = _weights_case("gauss", N, 256, seed=4)
    pb, gb = bl.quantize_weights(to_dev(Wb))
    pbr, gbr, _ = oracle.quantize_weights(Wb)
    packed_b = pb.unsqueeze(0).expand(B, N, 64).contiguous()
    gamma_b = gb.expand(B).contiguous()
    y = bl.forward_fused_batched(to_dev(Xb), packed_b, gamma_b, bits=bits, gran=gran,
                                 out_dtype=torch.int32)
    torch.cuda.synchronize()
    yh = to_host(y)
    for b in (0, 1, 2, 3):
        xq_b, s_b = oracle.quantize_acts(Xb[b], bits=bits, gran=g)
        _, acc_ref = oracle.forward(xq_b, bits, s_b, g, pbr, gbr, y_dtype=oracle.F32)
        assert_same_bytes(yh[b], acc_ref, "streamed accumulators problem %d" % b)


# batched fused forward: independent problems of one shape in one call
@pytest.mark.parametrize("B,M,K,N,bits,gran,epi,ydt,xdt,with_bias", [
    (3, 1, 256, 512, 8, "token", "relu2", "f32", "f32", True),
    (5, 5, 2560, 304, 4, "tensor", None, "bf16", "bf16", False),
    (2, 16, 640, 48, 8, "token", None, "i32", "bf16", False),
    (4, 1, 2560, 6912, 8, "token", "relu2", "bf16", "bf16", False),
    (4, 1, 6912, 2560, 8, "token", None, "bf16", "bf16", False),
    (2, 40, 256, 128, 8, "token", "relu2", "f32", "f32", True),  # one launch per problem
    # >= 2048 groups of 64 rows per launch: the streaming kernel
    (40, 1, 320, 4000, 8, "token", "relu2", "bf16", "bf16", False),  # ragged rows, partial k tile
    (36, 5, 256, 4096, 4, "tensor", None, "f32", "f32", True),
    (33, 16, 192, 4100, 8, "token", "relu2", "f32", "bf16", True),
    (64, 2, 64, 2048, 8, "token", None, "i32", "f32", False),
    # whole-line loads (K % 512 == 0), up to the 16-token limit
    (34, 3, 1024, 4000, 8, "token", "relu2", "bf16", "bf16", True),
    (33, 16, 512, 4100, 8, "token", None, "f32", "f32", False),
    # shifted whole-line loads (K % 512 == 256, at most 8 tokens): ragged last row tile
    # ending on an odd row and on an even row, both activation widths, int4 codes
    (36, 8, 768, 4003, 8, "token", "relu2", "f32", "bf16", True),
    (33, 7, 1280, 4004, 4, "tensor", None, "i32", "f32", False),
    (32, 1, 256, 4096, 4, "token", None, "bf16", "bf16", True),
    # 9 tokens at K % 512 == 256: the half-line loads
    (32, 9, 768, 4096, 8, "token", None, "bf16", "bf16", False),
])
def test_forward_fused_batched(B, M, K, N, bits, gran, epi, ydt, xdt, with_bias):
    say("forward_fused_batched", dict(B=B, M=M, K=K, N=N, bits=bits, gran=gran, epi=epi, y=ydt,
                                      x=xdt, bias=with_bias))
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    e = oracle.EPI_RELU2 if epi == "relu2" else oracle.EPI_NONE
    tdt, odt = YD[ydt]
    kind = "ternary" if N * K > 1 << 20 else "gauss"
    cases = [_layer(M, K, N, seed=10 + b, kind=kind) for b in range(B)]
    Xin = np.stack([workloads.to_bf16_bits(X) if xdt == "bf16" else X for _, X in cases])
    bias = (np.random.default_rng(B).standard_normal((B, N)).astype(np.float32)
            if with_bias else None)
    packed = torch.empty((B, N, K // 4), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((B,), dtype=torch.float32, device="cuda")
    for b, (W, _) in enumerate(cases):
        bl.quantize_weights(to_dev(W), out=(packed[b], gamma[b:b + 1]))
    y = bl.forward_fused_batched(to_dev(Xin), packed, gamma, bits=bits, gran=gran,
                                 bias=to_dev(bias) if with_bias else None, epilogue=epi,
                                 out_dtype=tdt)
    torch.cuda.synchronize()
    yh = to_host(y)
    for b, (W, _) in enumerate(cases):
        p_ref, g_ref, _ = oracle.quantize_weights(W)
        xq_ref, s_ref = oracle.quantize_acts(Xin[b], bits=bits, gran=g)
        y_ref, acc_ref = oracle.forward(xq_ref, bits, s_ref, g, p_ref, g_ref,
                                        bias=bias[b] if with_bias else None, epi=e,
                                        y_dtype=odt if odt is not None else oracle.F32)
        assert_y_matches(yh[b], acc_ref if ydt == "i32" else y_ref, ydt, "Y problem %d" % b)


# several projections of one quantized input in one call (a block's Q, K, V): part p
# against the oracle's forward of the shared codes with part p's weights
@pytest.mark.parametrize("P,M,K,N,bits,gran,epi,ydt,with_bias", [
    (3, 16, 2560, 2560, 8, "token", None, "bf16", False),   # the 2B block's Q, K, V
    (2, 1, 256, 512, 8, "token", "relu2", "f32", True),
    (4, 5, 640, 304, 4, "tensor", None, "i32", False),
    (2, 16, 6912, 2560, 8, "tensor", "relu2", "bf16", True),
    (3, 300, 256, 128, 8, "token", None, "f32", False),     # prefill-sized: one call per part
    (3, 2, 512, 44000, 8, "token", None, "bf16", False),    # >= 8192 row tiles: streaming
    (1, 3, 256, 128, 8, "token", None, "f32", False),       # a single part
    (2, 4, 256, 36, 8, "tensor", "relu2", "f32", True),     # ragged: 36 rows per part
])
def test_forward_multi(P, M, K, N, bits, gran, epi, ydt, with_bias):
    say("forward_multi", dict(P=P, M=M, K=K, N=N, bits=bits, gran=gran, epi=epi, y=ydt,
                              bias=with_bias))
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    e = oracle.EPI_RELU2 if epi == "relu2" else oracle.EPI_NONE
    tdt, odt = YD[ydt]
    kind = "ternary" if N * K > 1 << 20 else "gauss"
    X = _acts_case(M, K, seed=77)
    xq_ref, s_ref = oracle.quantize_acts(X, bits=bits, gran=g)
    Ws = [_weights_case(kind, N, K, seed=20 + p) for p in range(P)]
    bias = (np.random.default_rng(P).standard_normal((P, N)).astype(np.float32)
            if with_bias else None)
    packed = torch.empty((P, N, K // 4), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((P,), dtype=torch.float32, device="cuda")
    for p, W in enumerate(Ws):
        bl.quantize_weights(to_dev(W), out=(packed[p], gamma[p:p + 1]))
    y = bl.forward_multi(to_dev(xq_ref), to_dev(s_ref), packed, gamma, bits=bits, gran=gran,
                         bias=to_dev(bias) if with_bias else None, epilogue=epi, out_dtype=tdt)
    torch.cuda.synchronize()
    yh = to_host(y)
    for p, W in enumerate(Ws):
        p_ref, g_ref, _ = oracle.quantize_weights(W)
        assert_same_bytes(to_host(packed[p]), p_ref, "packed part %d" % p)
        if M * N * K > 3e8:
            ms, ns = sample_positions(M, N, 4096, p)
            y_ref, acc_ref = oracle.forward_at(xq_ref, bits, s_ref, g, p_ref, g_ref, ms, ns,
                                               bias=bias[p] if with_bias else None, epi=e,
                                               y_dtype=odt if odt is not None else oracle.F32)
            assert_y_matches(yh[p][ms, ns], acc_ref if ydt == "i32" else y_ref, ydt,
                             "Y part %d (sampled)" % p)
        else:
            y_ref, acc_ref = oracle.forward(xq_ref, bits, s_ref, g, p_ref, g_ref,
                                            bias=bias[p] if with_bias else None, epi=e,
                                            y_dtype=odt if odt is not None else oracle.F32)
            assert_y_matches(yh[p], acc_ref if ydt == "i32" else y_ref, ydt, "Y part %d" % p)


# one very wide layer (2048 groups of 64 rows): the streaming kernel on a single problem
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("fused", [False, True])
def test_forward_wide_stream(bits, fused):
    _check_forward(3, 64, 131072, bits, "token", "relu2", "f32", True, fused, sampled=False)
    _check_forward(1, 128, 131072 + 40, bits, "tensor", None, "i32", False, fused, sampled=False)


# the streamed decode step at full size, in the launch configuration the benchmark
# times: 64 2B-shaped layers per batched launch (streaming kernel); sampled problems
# are compared in full against the oracle
@pytest.mark.parametrize("shape,epi", [(workloads.SHAPE_UP, "relu2"), (workloads.SHAPE_DOWN, None)])
def test_forward_fused_batched_2b_64_layers(shape, epi):
    K, N = shape
    B = 64
    say("forward_fused_batched 64 layers", shape)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    codes = torch.randint(-1, 2, (B, N, K), device="cuda", generator=gen, dtype=torch.int8)
    packed = torch.empty((B, N, K // 4), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((B,), dtype=torch.float32, device="cuda")
    for b in range(B):
        bl.quantize_weights(codes[b].float(), out=(packed[b], gamma[b:b + 1]))
    X = torch.randn((B, 1, K), device="cuda", generator=gen).to(torch.bfloat16)
    y = bl.forward_fused_batched(X, packed, gamma, epilogue=epi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e = oracle.EPI_RELU2 if epi else oracle.EPI_NONE
    for b in (0, 1, 31, 63):
        W = codes[b].cpu().numpy().astype(np.float32)
        p_ref, g_ref, _ = oracle.quantize_weights(W)
        assert_same_bytes(to_host(packed[b]), p_ref, "packed layer %d" % b)
        y_ref, _, _, _ = oracle.bitlinear(to_host(X[b]), p_ref, g_ref, epi=e, y_dtype=oracle.BF16)
        assert_same_bytes(to_host(y[b]), y_ref, "Y layer %d" % b)


# streamed launches of a few tokens with long rows in all three load modes -- whole
# lines (K % 512 == 0), shifted whole lines (K % 512 == 256) and half lines with a
# partial last k tile; device-drawn uniform-ternary codes, sampled problems compared in
# full against the oracle (their packing first against the oracle's)
@pytest.mark.parametrize("B,M,K,N,bits,gran,epi,ydt,with_bias", [
    (32, 2, 4096, 4096, 8, "token", "relu2", "bf16", True),
    (32, 3, 4864, 4096, 4, "tensor", None, "i32", False),
    (32, 4, 4416, 4096, 8, "token", None, "f32", False),
    (64, 4, 6912, 2560, 8, "tensor", "relu2", "bf16", True),
])
def test_forward_stream_long_rows(B, M, K, N, bits, gran, epi, ydt, with_bias):
    say("stream long rows", dict(B=B, M=M, K=K, N=N, bits=bits, gran=gran, epi=epi, y=ydt,
                                 bias=with_bias))
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    e = oracle.EPI_RELU2 if epi == "relu2" else oracle.EPI_NONE
    tdt, odt = YD[ydt]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(B * 7 + K)
    packed = torch.empty((B, N, K // 4), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((B,), dtype=torch.float32, device="cuda")
    sampled = (0, 1, B // 2, B - 1)
    host_codes = {}
    for b in range(B):
        codes = torch.randint(-1, 2, (N, K), device="cuda", generator=gen, dtype=torch.int8)
        bl.quantize_weights(codes.float(), out=(packed[b], gamma[b:b + 1]))
        if b in sampled:
            host_codes[b] = codes.cpu().numpy().astype(np.float32)
    X = torch.randn((B, M, K), device="cuda", generator=gen).to(torch.bfloat16)
    bias = torch.randn((B, N), device="cuda", generator=gen) if with_bias else None
    y = bl.forward_fused_batched(X, packed, gamma, bits=bits, gran=gran, bias=bias, epilogue=epi,
                                 out_dtype=tdt)
    torch.cuda.synchronize()
    for b in sampled:
        p_ref, g_ref, _ = oracle.quantize_weights(host_codes[b])
        assert_same_bytes(to_host(packed[b]), p_ref, "packed problem %d" % b)
        y_ref, acc_ref, _, _ = oracle.bitlinear(to_host(X[b]), p_ref, g_ref, bits=bits, gran=g,
                                                bias=to_host(bias[b]) if with_bias else None, epi=e,
                                                y_dtype=odt if odt is not None else oracle.F32)
        assert_y_matches(to_host(y[b]), acc_ref if ydt == "i32" else y_ref, ydt, "Y problem %d" % b)


# maximum sizes: one layer at the ABI's limit N*K < 2^32 (65535 x 65536, 8.6 GB of bf16
# weights on the device); gamma against its exact value nnz/(NK), outputs of sampled
# rows against the oracle (the codes of uniform-ternary weights are the weights)
def test_max_size_layer():
    from fractions import Fraction
    from exact import round_to_f32
    N, K = 65535, 65536
    assert N * K < 1 << 32
    say("max-size layer", N, K)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    codes = torch.randint(-1, 2, (N, K), device="cuda", generator=gen, dtype=torch.int8)
    nnz = int(torch.count_nonzero(codes))
    W = codes.to(torch.bfloat16)
    packed, gamma = bl.quantize_weights(W)
    del W
    torch.cuda.synchronize()
    g_ref = round_to_f32(Fraction(nnz, N * K))
    assert bits32(to_host(gamma))[0] == bits32(np.array([g_ref]))[0], "gamma differs"
    rows = np.array([0, 1, 12345, 40000, N - 2, N - 1])
    c_rows = codes[torch.from_numpy(rows).cuda()].cpu().numpy()
    # the packed rows are the codes, re-packed by the oracle's own packer
    p_rows, _, _ = oracle.quantize_weights(c_rows.astype(np.float32))
    assert_same_bytes(to_host(packed[torch.from_numpy(rows).cuda()]), p_rows, "packed rows")
    del codes
    for M in (1, 300):
        rng = np.random.default_rng(M)
        X = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        say("max-size forward", M)
        y = bl.forward_fused(to_dev(X), packed, gamma, out_dtype=torch.float32)
        torch.cuda.synchronize()
        xq_ref, s_ref = oracle.quantize_acts(X)
        ms = np.repeat(np.arange(M)[[0, M // 2, M - 1]], len(rows))
        ns_local = np.tile(np.arange(len(rows)), 3)
        y_ref, _ = oracle.forward_at(xq_ref, 8, s_ref, oracle.PER_TOKEN, p_rows, g_ref,
                                     ms, ns_local, y_dtype=oracle.F32)
        got = to_host(y)[ms, rows[ns_local]]
        assert_y_matches(got, y_ref, "f32", "Y max-size M=%d" % M)
        del y
