"""Seeded synthetic inputs for the BitLinear workloads.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, packing, contraction or rescale), so
both the oracle and the HIP path can be fed from it.  bf16 inputs are made by
torch's float32 -> bfloat16 conversion (round to nearest even) and returned as
``numpy.uint16`` bit patterns.

The shapes and value statistics follow the pages' models: the BitNet b1.58
2B4T layer shapes (hidden 2560, FFN 6912, 30 blocks; "BitNet 2B4T Guide",
"End-to-End PyTorch Implementation" gives the block structure) and a 70B-class
FFN layer (K=8192, N=28672) for the a4.8 INT4-vs-INT8 comparison ("BitNet a4.8
Guide", "The Activation Bottleneck" on outlier channels).  No trained weights
or datasets are used: weights are drawn, and activations are Gaussian with a
few scaled outlier channels.
"""
from __future__ import annotations

import numpy as np
import torch

HIDDEN = 2560
FFN = 6912
LAYERS_2B = 30
QKV = 3 * HIDDEN

# (K, N) pairs of the two FFN projections of the 2B model
SHAPE_UP = (HIDDEN, FFN)     # 2560 -> 6912, ReLU^2 applied on its output
SHAPE_DOWN = (FFN, HIDDEN)   # 6912 -> 2560

SHAPE_70B = (8192, 28672)    # (K, N) of the 70B-class FFN layer


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ternary_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """float32 [n, k] with entries drawn uniformly from {-1, 0, +1}."""
    return rng.integers(-1, 2, size=(n, k), dtype=np.int8).astype(np.float32)


def ternary_codes(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 [n, k] with entries drawn uniformly from {-1, 0, +1}."""
    return rng.integers(-1, 2, size=(n, k), dtype=np.int8)


def outlier_acts(rng: np.random.Generator, m: int, k: int, n_outliers: int,
                 factor: float) -> np.ndarray:
    """float32 [m, k] ~ N(0,1) with ``n_outliers`` channels scaled by ``factor``."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if n_outliers:
        idx = rng.choice(k, n_outliers, replace=False)
        x[:, idx] *= np.float32(factor)
    return x


def parity_layer(seed: int = 0, m: int = 8, k: int = 256, n: int = 512):
    """Small single-layer case: W = 0.02 * N(0,1) [n, k] fp32, X = N(0,1) [m, k] fp32
    with 4 outlier channels x20.  Draw order: W, X, outlier indices."""
    rng = np.random.default_rng(seed)
    W = (np.float32(0.02) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    X = rng.standard_normal((m, k), dtype=np.float32)
    idx = rng.choice(k, 4, replace=False)
    X[:, idx] *= np.float32(20.0)
    return W, X


def decode_gemv(seed: int = 1, shape=SHAPE_UP, m: int = 1):
    """Decode GEMV case: W uniform ternary as float32 [N, K]; x ~ N(0,1) [m, K] as bf16."""
    k, n = shape
    rng = np.random.default_rng([seed, k, n])
    W = ternary_weights(rng, n, k)
    x = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    return W, x


def prefill_gemm(seed: int = 2, shape=SHAPE_UP, m: int = 2048):
    """Prefill GEMM case: W uniform ternary float32 [N, K]; X ~ N(0,1) [m, K] as bf16."""
    k, n = shape
    rng = np.random.default_rng([seed, k, n])
    W = ternary_weights(rng, n, k)
    X = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    return W, X


def stack_layer_codes(seed: int, layer: int):
    """Ternary codes of one block of the 30-layer 2B stack, each projection drawn from
    its own stream so any layer can be regenerated alone.
    Returns dict name -> int8 [N, K] for qkv [7680, 2560], o [2560, 2560],
    up [6912, 2560], down [2560, 6912]."""
    out = {}
    for j, (name, n, k) in enumerate((("qkv", QKV, HIDDEN), ("o", HIDDEN, HIDDEN),
                                      ("up", FFN, HIDDEN), ("down", HIDDEN, FFN))):
        rng = np.random.default_rng([seed, layer, j])
        out[name] = ternary_codes(rng, n, k)
    return out


def stack_input(seed: int = 3, m: int = 16):
    """x0 ~ N(0,1) [m, 2560] as bf16 for the 30-layer stack."""
    rng = np.random.default_rng([seed, 1 << 20])
    return to_bf16_bits(rng.standard_normal((m, HIDDEN), dtype=np.float32))


def layer_70b(seed: int = 4, m: int = 4096, shape=SHAPE_70B, outlier_frac: float = 0.005,
              factor: float = 30.0):
    """70B-class FFN layer: W uniform ternary codes int8 [N, K]; X ~ N(0,1) [m, K] with
    round(outlier_frac * K) outlier channels x factor, as bf16."""
    k, n = shape
    rng = np.random.default_rng([seed, k, n])
    codes = ternary_codes(rng, n, k)
    n_out = int(round(outlier_frac * k))
    X = to_bf16_bits(outlier_acts(rng, m, k, n_out, factor))
    return codes, X


def random_case(seed: int, m: int, k: int, n: int, w_scale: float = 0.02,
                x_scale: float = 1.0, n_outliers: int = 0, factor: float = 20.0):
    """Generic Gaussian case for parity sweeps (fp32 W and X)."""
    rng = np.random.default_rng([seed, m, k, n])
    W = (np.float32(w_scale) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    X = (np.float32(x_scale) * outlier_acts(rng, m, k, n_outliers, factor)).astype(np.float32)
    return W, X
