"""GPU parity of the balanced-tile prefill GEMM (csrc/gemm_mid.hip, the 16 x 16 x 64 int8
matrix cores): 128 x 160 tiles (four-wave groups) and 128 x 448 tiles (eight waves).
The large-tile launcher hands a shape to them when their tiles leave each CU at most
three quarters (128 x 160) or nine tenths (128 x 448) of the large tiles' work: every
shape below is one of those (among them the 2B down projection at 2048 tokens, 256
tiles of 128 x 160 exactly, whose full int32 accumulators test_parity_gpu.py checks,
and the 2B up projection, 256 tiles of 128 x 448).

"BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free Forward
Pass & Dequantization": int32 accumulators and every output bit-exact against the
oracle, element by element: ragged M and N (partial tiles in both directions), one k
step, odd and even numbers of them, K a multiple of 128 (two k steps per LDS stage) or
not, more tiles than CUs; every epilogue and output type; per-token and per-tensor
scales."""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import say
from test_parity_gpu import _check_forward, _codes_f64, _layer, _run_forward

pytestmark = pytest.mark.gpu

# (M, K, N)
MID_SHAPES = [(128, 64, 128), (129, 64, 130), (300, 192, 257), (1000, 384, 700),
              (513, 576, 900), (2048, 128, 4096)]


@pytest.mark.parametrize("M,K,N", MID_SHAPES)
@pytest.mark.parametrize("fused", [False, True])
def test_mid_shapes(M, K, N, fused):
    _check_forward(M, K, N, 8, "token", None, "i32", False, fused, sampled=False)
    _check_forward(M, K, N, 8, "token", "relu2", "bf16", False, fused, sampled=False, seed=1,
                   x_dtype="bf16")


@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("epi", [None, "relu2"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("K", [320, 256])
def test_mid_variants(gran, epi, ydt, with_bias, K):
    # N % 8 != 0 (bf16 stored from registers) and N % 8 == 0 (bf16 staged through LDS and
    # stored in whole 16-byte chunks), each with a partial last row block
    _check_forward(300, K, 260, 8, gran, epi, ydt, with_bias, False, sampled=False)
    _check_forward(300, K, 264, 8, gran, epi, ydt, with_bias, False, sampled=False, seed=5)


@pytest.mark.parametrize("K", [320, 384])
def test_mid_more_tiles_than_cus(K):
    # 17 x 25 = 425 tiles: two blocks on some CUs; outputs sampled, then the full int32
    # accumulators against a float64 product of the oracle's codes (exact: integers
    # below 2^53)
    M, N = 2100, 4000
    _check_forward(M, K, N, 8, "token", "relu2", "bf16", True, True, x_dtype="bf16",
                   kind="ternary", sampled=True)
    W, X = _layer(M, K, N, 0, "ternary")
    say("mid GEMM, full int32 accumulators", M, K, N)
    acc, (p_ref, _, xq_ref, _, _) = _run_forward(W, X, 8, "token", None, "i32", None, False, "bf16")
    q, c = _codes_f64(xq_ref, 8, p_ref, K)
    assert np.array_equal(acc.astype(np.float64), q @ c.T), "int32 accumulators differ"


# 128 x 448 tiles: about one tile per CU where 256 x 256 tiles would leave CUs idle
WIDE_SHAPES = [(1024, 64, 14336), (1900, 128, 7000), (2000, 192, 6900)]


@pytest.mark.parametrize("M,K,N", WIDE_SHAPES)
def test_wide_shapes(M, K, N):
    _check_forward(M, K, N, 8, "token", None, "i32", False, False, sampled=False)
    _check_forward(M, K, N, 8, "token", "relu2", "bf16", True, True, sampled=False, seed=1,
                   x_dtype="bf16")


@pytest.mark.parametrize("gran", ["token", "tensor"])
@pytest.mark.parametrize("epi", [None, "relu2"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_wide_variants(gran, epi, ydt, with_bias):
    _check_forward(1024, 64, 14336, 8, gran, epi, ydt, with_bias, False, sampled=False)


# the 2B up projection at 2048 tokens (40 k steps, two per stage), a ragged shape with an
# odd number of single k steps, and two rounds of tiles (496 tiles): outputs sampled, then
# the full int32 accumulators against a float64 product of the oracle's codes
@pytest.mark.parametrize("M,K,N", [(2048, 2560, 6912), (2000, 2496, 6900), (2048, 256, 13824)])
def test_wide_accumulators(M, K, N):
    _check_forward(M, K, N, 8, "token", "relu2", "bf16", True, True, x_dtype="bf16",
                   kind="ternary", sampled=True)
    W, X = _layer(M, K, N, 0, "ternary")
    say("wide GEMM, full int32 accumulators", M, K, N)
    acc, (p_ref, _, xq_ref, _, _) = _run_forward(W, X, 8, "token", None, "i32", None, False, "bf16")
    q, c = _codes_f64(xq_ref, 8, p_ref, K)
    assert np.array_equal(acc.astype(np.float64), q @ c.T), "int32 accumulators differ"
