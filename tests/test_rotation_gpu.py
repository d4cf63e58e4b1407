"""GPU parity of the Hadamard rotation folded into the quantizers ("BitNet a4.8 Guide",
"Best Practices for Deploying BitNet a4.8 in Production", Outlier Suppression row):
bitlinear_quantize_acts_rotated and bitlinear_quantize_weights_rotated against the
oracle, bit for bit (the rotation is a fixed fp32 operation order on both sides), and
the forward on rotated operands.
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


def _acts(m, k, seed, outliers=True):
    rng = np.random.default_rng([seed, m, k])
    X = rng.standard_normal((m, k)).astype(np.float32)
    if outliers:
        X[:, rng.choice(k, max(1, k // 200), replace=False)] *= 30.0
    return X


@pytest.mark.parametrize("m,k", [(8, 256), (3, 2560), (5, 6912), (4, 8192), (2, 16384), (7, 48),
                                 (1, 16)])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_acts_rotated_parity(m, k, bits, gran, dtype):
    X = _acts(m, k, 1)
    Xin = workloads.to_bf16_bits(X) if dtype == "bf16" else X
    say("quantize_acts_rotated", m, k, bits, gran, dtype)
    xq, s = bl.quantize_acts_rotated(to_dev(Xin), bits=bits, gran=gran)
    torch.cuda.synchronize()
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts_rotated(Xin, bits=bits, gran=g)
    assert_same_bytes(bits32(to_host(s)), bits32(s_ref), "act_scale")
    assert_same_bytes(to_host(xq), xq_ref, "rotated activation codes")


def _weights(kind, n, k, seed=0):
    rng = np.random.default_rng([seed, n, k])
    if kind == "gauss":
        return (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    if kind == "ternary":
        return workloads.ternary_weights(rng, n, k)
    if kind == "zeros":
        return np.zeros((n, k), np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind,n,k,dtype", [
    ("gauss", 64, 256, "f32"), ("gauss", 33, 2560, "bf16"), ("gauss", 128, 6912, "f32"),
    ("ternary", 64, 8192, "f32"), ("gauss", 16, 16384, "f32"), ("zeros", 8, 512, "f32"),
    ("gauss", 1500, 48, "f32"), ("gauss", 2048, 2560, "f32"),
])
def test_quantize_weights_rotated_parity(kind, n, k, dtype):
    W = _weights(kind, n, k)
    Win = workloads.to_bf16_bits(W) if dtype == "bf16" else W
    say("quantize_weights_rotated", kind, n, k, dtype)
    packed, gamma = bl.quantize_weights_rotated(to_dev(Win))
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights_rotated(Win)
    assert bits32(to_host(gamma))[0] == bits32(np.array([g_ref]))[0], "gamma differs"
    assert_same_bytes(to_host(packed), p_ref, "rotated packed weights")


@pytest.mark.parametrize("M,K,N,bits", [(8, 256, 512, 8), (8, 256, 512, 4), (300, 2560, 384, 4),
                                        (300, 2560, 384, 8), (1, 6912, 2560, 8), (16, 8192, 300, 4)])
def test_forward_on_rotated_operands(M, K, N, bits):
    X = _acts(M, K, 2)
    W = _weights("gauss", N, K, 3)
    say("forward rotated", M, K, N, bits)
    packed, gamma = bl.quantize_weights_rotated(to_dev(W))
    xq, s = bl.quantize_acts_rotated(to_dev(X), bits=bits)
    y = bl.forward(xq, s, packed, gamma, bits=bits, out_dtype=torch.float32)
    acc = bl.forward(xq, s, packed, gamma, bits=bits, out_dtype=torch.int32)
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights_rotated(W)
    xq_ref, s_ref = oracle.quantize_acts_rotated(X, bits=bits)
    y_ref, acc_ref = oracle.forward(xq_ref, bits, s_ref, oracle.PER_TOKEN, p_ref, g_ref)
    assert_same_bytes(to_host(acc), acc_ref, "acc")
    assert_y_matches(to_host(y), y_ref, "f32", "Y")


def test_rotated_70b_layer_sampled():
    # the 70B-class layer's shapes and outliers, float master weights: rotated int4
    # codes, gamma and sampled outputs against the oracle
    rng = np.random.default_rng(4)
    M, K, N = 4096, 8192, 28672
    W = (0.02 * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)
    _, X = workloads.layer_70b()
    say("rotated 70B layer", M, K, N)
    packed, gamma = bl.quantize_weights_rotated(to_dev(W))
    Xd = to_dev(X)
    xq, s = bl.quantize_acts_rotated(Xd, bits=4)
    y = bl.forward(xq, s, packed, gamma, bits=4, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights_rotated(W)
    del W
    assert bits32(to_host(gamma))[0] == bits32(np.array([g_ref]))[0], "gamma differs"
    assert_same_bytes(to_host(packed), p_ref, "rotated packed weights (all rows)")
    xq_ref, s_ref = oracle.quantize_acts_rotated(X, bits=4)
    assert_same_bytes(bits32(to_host(s)), bits32(s_ref), "act_scale")
    assert_same_bytes(to_host(xq), xq_ref, "rotated int4 codes")
    ms, ns = sample_positions(M, N, 2048, 5)
    y_ref, _ = oracle.forward_at(xq_ref, 4, s_ref, oracle.PER_TOKEN, p_ref, g_ref, ms, ns,
                                 y_dtype=oracle.BF16)
    assert_y_matches(to_host(y)[ms, ns], y_ref, "bf16", "Y rotated (sampled)")
