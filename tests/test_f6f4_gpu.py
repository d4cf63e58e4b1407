"""GPU parity of the 4-bit-activation prefill path, which runs on the FP6 x FP4 scaled
matrix cores (bits=4, M >= 128, N >= 128, K % 64 == 0, K < 2^20).

The int4 codes enter the MFMA as q/2 in e2m3 and the ternary fields as (c+1)/2 in
e2m1; the claim is that the fp32 accumulation is then exact, so the path must match
the oracle's integer contraction to the bit:
- element by element at ragged shapes on every tile shape, every epilogue and output;
- closed forms at the largest K the path takes (2^20 - 64), where the accumulator sits
  at 4K, the edge of exact fp32: all codes -8 against c = +1 must give exactly -8K;
- sampled oracle outputs for random codes at that K, and the same closed forms at
  K = 2^20, where the int8 path takes over.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import DEV, assert_same_bytes, say, to_dev, to_host
from test_parity_gpu import _check_forward, _codes_f64, _layer, _run_forward

pytestmark = pytest.mark.gpu

K_MAX_F6 = (1 << 20) - 64

# (M, K, N): one tile, ragged M and N, several k steps; 128-wide tiles (few tiles),
# 256-wide tiles (at least 128 tiles of 256 x 256) with one k step, an even and two odd
# numbers of them, and with two k steps per LDS stage where K % 128 == 0 (3000 x 384 x
# 4000: three stages, ragged); and, where K % 128 == 0 and they leave fewer CUs idle, the
# balanced 128 x 160 tiles on the 16 x 16 x 128 MFMA (one wave group: 129 x 128 x 130,
# 513 x 640 x 1000, 2048 x 128 x 4096; two on alternate stages: 256 x 2560 x 384)
F6_SHAPES = [(128, 64, 128), (129, 128, 130), (300, 192, 257), (256, 2560, 384),
             (513, 640, 1000), (2048, 128, 4096), (2048, 64, 4096), (2100, 320, 4000),
             (2304, 448, 3900), (3000, 384, 4000)]


@pytest.mark.parametrize("M,K,N", F6_SHAPES)
@pytest.mark.parametrize("fused", [False, True])
def test_f6f4_shapes(M, K, N, fused):
    _check_forward(M, K, N, 4, "token", None, "i32", False, fused, sampled=False)
    _check_forward(M, K, N, 4, "token", "relu2", "bf16", False, fused, sampled=False, seed=1)


@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("epi", [None, "relu2"])
@pytest.mark.parametrize("ydt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_f6f4_variants(gran, epi, ydt, with_bias):
    if ydt == "i32" and (epi or with_bias):
        pytest.skip("raw accumulators take no epilogue")
    # 256-row tiles (K = 320); balanced 128 x 160 tiles with one wave group (K = 384) and
    # with two on alternate k stages (K = 256)
    _check_forward(300, 320, 260, 4, gran, epi, ydt, with_bias, False, sampled=False)
    _check_forward(300, 384, 260, 4, gran, epi, ydt, with_bias, False, sampled=False, seed=3)
    _check_forward(257, 256, 388, 4, gran, epi, ydt, with_bias, True, x_dtype="bf16",
                   sampled=False, seed=2)
    # the same two balanced forms with N % 8 == 0 (bf16 staged through LDS, whole chunks)
    _check_forward(300, 384, 264, 4, gran, epi, ydt, with_bias, False, sampled=False, seed=6)
    _check_forward(257, 256, 392, 4, gran, epi, ydt, with_bias, True, x_dtype="bf16",
                   sampled=False, seed=7)
    # 256-row tiles with two k steps per LDS stage, 256 tiles (outputs sampled)
    _check_forward(1024, 128, 14336, 4, gran, epi, ydt, with_bias, False, sampled=True, seed=4)


# Larger shapes on the 256-row tiles with two k steps per LDS stage: outputs sampled,
# then the full int32 accumulators against a float64 product of the oracle's codes
# (exact: integers below 2^53).  The 2B up projection at 2048 tokens (216 tiles), two
# rounds of tiles (432), and ragged shapes with 256 tiles and with an odd number of
# stages.
@pytest.mark.parametrize("M,K,N", [(2048, 2560, 6912), (2048, 256, 13824), (2000, 256, 6900),
                                   (2000, 384, 8100)])
def test_f6f4_accumulators(M, K, N):
    _check_forward(M, K, N, 4, "token", "relu2", "bf16", True, True, x_dtype="bf16",
                   kind="ternary", sampled=True)
    W, X = _layer(M, K, N, 0, "ternary")
    say("FP6 x FP4 GEMM, full int32 accumulators", M, K, N)
    acc, (p_ref, _, xq_ref, _, _) = _run_forward(W, X, 4, "token", None, "i32", None, False, "bf16")
    q, c = _codes_f64(xq_ref, 4, p_ref, K)
    assert np.array_equal(acc.astype(np.float64), q @ c.T), "int32 accumulators differ"


def _const_case(M, N, K, qbyte, wbyte):
    xq = torch.full((M, K // 2), qbyte, dtype=torch.uint8, device=DEV)
    packed = torch.full((N, K // 4), wbyte, dtype=torch.uint8, device=DEV)
    s = torch.ones(M, dtype=torch.float32, device=DEV)
    gamma = torch.ones(1, dtype=torch.float32, device=DEV)
    return xq, s, packed, gamma


# int4 byte (two equal codes) x packed weight byte (four equal fields) -> acc / K
EXTREMES = [(0x88, 0xAA, -8),   # q = -8, c = +1
            (0x88, 0x00, 8),    # q = -8, c = -1
            (0x77, 0x00, -7),   # q = +7, c = -1
            (0x77, 0xAA, 7),    # q = +7, c = +1
            (0x99, 0x55, 0)]    # q = -7, c = 0


@pytest.mark.parametrize("K", [K_MAX_F6, 1 << 20])
@pytest.mark.parametrize("qbyte,wbyte,per_k", EXTREMES)
def test_f6f4_extreme_codes_largest_k(K, qbyte, wbyte, per_k):
    M, N = 128, 160
    say("f6f4 extremes", dict(K=K, q=hex(qbyte), w=hex(wbyte)))
    xq, s, packed, gamma = _const_case(M, N, K, qbyte, wbyte)
    acc = bl.forward(xq, s, packed, gamma, bits=4, out_dtype=torch.int32)
    y = bl.forward(xq, s, packed, gamma, bits=4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = to_host(acc)
    assert (a == per_k * K).all(), (int(a.min()), int(a.max()), per_k * K)
    # f = s * gamma = 1, so y = (float)acc exactly (|acc| <= 2^23)
    assert (to_host(y) == np.float32(per_k * K)).all()


def test_f6f4_random_codes_largest_k():
    M, N, K = 160, 136, K_MAX_F6
    rng = np.random.default_rng(11)
    xq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)        # every int4 code, -8 included
    f = rng.integers(0, 3, (N, K), dtype=np.uint8)                  # fields c + 1
    packed = (f[:, 0::4] | (f[:, 1::4] << 2) | (f[:, 2::4] << 4) | (f[:, 3::4] << 6)).astype(np.uint8)
    del f
    s = (rng.random(M, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    gamma = np.array([0.75], np.float32)
    say("f6f4 random codes", dict(M=M, N=N, K=K))
    d = (to_dev(xq), to_dev(s), to_dev(packed), to_dev(gamma))
    acc = bl.forward(*d, bits=4, out_dtype=torch.int32)
    y = bl.forward(*d, bits=4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ms = np.concatenate([np.arange(M), np.zeros(N, np.int64) + M - 1])
    ns = np.concatenate([np.arange(M) % N, np.arange(N)])
    y_ref, acc_ref = oracle.forward_at(xq, 4, s, oracle.PER_TOKEN, packed, gamma[0], ms, ns,
                                       y_dtype=oracle.F32)
    assert_same_bytes(to_host(acc)[ms, ns], acc_ref, "acc (sampled)")
    assert_same_bytes(to_host(y)[ms, ns], y_ref, "Y (sampled)")
