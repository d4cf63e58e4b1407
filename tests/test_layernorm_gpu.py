"""GPU parity of the non-affine layer norm before the quantizer ("BitNet b1.58: The 1-Bit
Ternary LLM Architecture Guide", "Implementation", Step 2 BitLinear listing), alone, fused
with the activation quantizer, and as the input side of a whole BitLinear.  Every result
is compared with the oracle's bit for bit: the row sums are exact on both sides, so no
reduction order can move a bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, assert_y_matches, bits32, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _rows(kind, rng, M, K):
    """bf16 rows of the named kind:
    gauss   N(0, 3^2)
    offset  N(40, 1): a large mean, small spread (the variance is a small difference)
    wide    N(0, 1) with a twentieth scaled by 2^-50 (below the window: the exact sums'
            slow path), a few subnormals and zeros
    cancel  each row holds x and -x (S1 = 0 exactly)
    const   one value per row (variance 0: h = 0)"""
    if kind == "gauss":
        x = 3.0 * rng.standard_normal((M, K))
    elif kind == "offset":
        x = 40.0 + rng.standard_normal((M, K))
    elif kind == "wide":
        x = rng.standard_normal((M, K)).astype(np.float32)
        x[rng.random((M, K)) < 0.05] *= np.float32(2.0 ** -50)
        sub = rng.random((M, K)) < 0.01
        x[sub] = np.float32(2.0 ** -130) * rng.integers(1, 64, size=int(sub.sum())).astype(np.float32)
        x[rng.random((M, K)) < 0.01] = 0.0
    elif kind == "cancel":
        half = rng.standard_normal((M, K // 2))
        x = np.concatenate([half, -half], axis=1)
        for r in x:
            rng.shuffle(r)
    else:
        x = np.repeat(rng.standard_normal((M, 1)) * 5.0, K, axis=1)
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("M,K,kind,with_delta", [
    (16, 2560, "gauss", True), (16, 2560, "offset", False), (3, 6912, "gauss", False),
    (5, 4104, "offset", True), (1, 8, "gauss", False), (2, 65536, "gauss", True),
    (7, 2560, "wide", False), (3, 4104, "wide", True), (2, 65536, "wide", False),
    (4, 2560, "cancel", False), (4, 96, "const", False), (9, 8192, "offset", False)])
def test_layernorm_parity(M, K, kind, with_delta):
    rng = np.random.default_rng([41, M, K, len(kind)])
    x = _rows(kind, rng, M, K)
    dlt = _rows("wide" if kind == "wide" else "gauss", rng, M, K) if with_delta else None
    say("layernorm", M, K, kind, with_delta)
    xd = to_dev(x)
    h = bl.layernorm(xd, to_dev(dlt) if with_delta else None)
    torch.cuda.synchronize()
    x_ref, h_ref = oracle.layernorm(x, dlt)
    assert_same_bytes(to_host(xd), x_ref, "layernorm %dx%d %s residual" % (M, K, kind))
    assert_same_bytes(to_host(h), h_ref, "layernorm %dx%d %s h" % (M, K, kind))
    if kind == "const":
        assert not to_host(h).any()


def test_layernorm_eps():
    # eps is the caller's: a row of spread 2^-10 against eps 1e-5 and 1e-2
    rng = np.random.default_rng(42)
    x = workloads.to_bf16_bits((2.0 ** -10 * rng.standard_normal((4, 512))).astype(np.float32))
    for eps in (1e-5, 1e-2):
        say("layernorm eps", eps)
        h = bl.layernorm(to_dev(x), eps=eps)
        torch.cuda.synchronize()
        assert_same_bytes(to_host(h), oracle.layernorm(x, eps=eps)[1], "eps %g" % eps)


@pytest.mark.parametrize("M,K,bits,gran,kind,with_delta", [
    (16, 2560, 8, "token", "gauss", True), (16, 6912, 8, "token", "offset", False),
    (3, 256, 4, "token", "gauss", True), (5, 4096, 8, "tensor", "offset", True),
    (2, 65536, 8, "token", "gauss", False), (1, 16, 4, "tensor", "gauss", False),
    (6, 2560, 8, "token", "wide", False), (4, 6912, 4, "token", "wide", True),
    (3, 2560, 4, "tensor", "cancel", False)])
def test_layernorm_quantize_parity(M, K, bits, gran, kind, with_delta):
    rng = np.random.default_rng([43, M, K, bits, len(kind)])
    x = _rows(kind, rng, M, K)
    dlt = _rows("gauss", rng, M, K) if with_delta else None
    say("layernorm_quantize", M, K, bits, gran, kind, with_delta)
    xd = to_dev(x)
    h, xq, sc = bl.layernorm_quantize(xd, to_dev(dlt) if with_delta else None, bits=bits,
                                      gran=gran)
    torch.cuda.synchronize()
    x_ref, h_ref = oracle.layernorm(x, dlt)
    assert_same_bytes(to_host(xd), x_ref, "residual")
    assert_same_bytes(to_host(h), h_ref, "h")
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts(h_ref, bits=bits, gran=g)
    assert_same_bytes(to_host(xq), xq_ref, "codes")
    assert_same_bytes(bits32(to_host(sc)), bits32(s_ref), "scales")


@pytest.mark.parametrize("M,K,N,bits", [(16, 2560, 6912, 8), (5, 6912, 2560, 8),
                                        (64, 2560, 2560, 4), (257, 512, 384, 8)])
def test_step2_bitlinear_chain(M, K, N, bits):
    """The Step 2 BitLinear end to end: layer norm -> absmax quantizer -> ternary weights
    (absmean) -> integer matmul -> rescale by gamma / s, with the GPU's calls against the
    oracle's chain from the same input and latent weights."""
    rng = np.random.default_rng([44, M, K, N, bits])
    x = workloads.to_bf16_bits((0.5 + 2.0 * rng.standard_normal((M, K))).astype(np.float32))
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    say("step2 chain", M, K, N, bits)
    packed, gamma = bl.quantize_weights(to_dev(W))
    h, xq, sc = bl.layernorm_quantize(to_dev(x), bits=bits)
    y = bl.forward(xq, sc, packed, gamma, bits=bits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    _, h_ref = oracle.layernorm(x)
    xq_ref, s_ref = oracle.quantize_acts(h_ref, bits=bits)
    y_ref, _ = oracle.forward(xq_ref, bits, s_ref, oracle.PER_TOKEN, p_ref, g_ref)
    assert_same_bytes(to_host(packed), p_ref, "packed")
    assert_same_bytes(to_host(h), h_ref, "h")
    assert_same_bytes(to_host(xq), xq_ref, "codes")
    assert_y_matches(to_host(y), y_ref, "f32", "y")
