"""CPU oracle for the BitLinear forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
(``ternary_weight_quantized_bitlinear_amd``) never imports it; the two share no
code.  The arithmetic lives in ``bitlinear_oracle.c`` (plain single-threaded C,
built with ``-ffp-contract=off``); this module only marshals numpy arrays.

Functions and the passages they follow (page titles abbreviated as in the C
source header):

* :func:`gamma` -- mean |W| ([b158] "The Mathematical Formulation of
  BitLinear", eq. 1), exact sum, rounded once to fp32, clamp(min=eps).
* :func:`quantize_weights` -- Clip(Round(W/gamma), -1, 1) and the 2-bit
  packing ([b158] eq. 1; [2b4t] "1. The BitLinear Operator").
* :func:`quantize_acts` -- per-token / per-tensor absmax int8 ([b158] eq. 2;
  [2b4t] "1. The BitLinear Operator") and int4 ([a48] "1. Hybrid W1.58 / A4
  Quantization Function").
* :func:`forward`, :func:`forward_at` -- integer contraction, rescale
  ([b158] eq. 3; [a48] dataflow figure), bias, ReLU^2 ([2b4t] "2. Squared
  ReLU Activation").
* :func:`backward` -- the layer's gradients under the straight-through estimators:
  int8 per [b158] "Implementation" Step 1-2 listings (identity STE, y = linear(q, c)
  * gamma/s), int4 per [a48] "Implementation" Step 2-3 listings (masked STE, y =
  linear(q s, c gamma)); fp64 sums of the fp32 operands the listings materialize.
* :func:`hadamard_block`, :func:`hadamard_rows`, :func:`quantize_acts_rotated`,
  :func:`quantize_weights_rotated` -- the Hadamard rotation folded into both
  operands before the 4-bit activation quantization ([a48] "Best Practices for
  Deploying BitNet a4.8 in Production", Outlier Suppression row): block-diagonal
  Sylvester blocks on the K axis, unnormalized fp32 fast transform, 1/b in gamma.

bf16 arrays are passed as ``numpy.uint16`` holding the bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
PER_TOKEN, PER_TENSOR = 0, 1
EPI_NONE, EPI_RELU2 = 0, 1


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB points the pin suite at a deliberately broken build (mutation tests)
        lib = ctypes.CDLL(os.environ.get("ORACLE_LIB") or build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        lib.oracle_gamma.argtypes = [P, I, I64, I64, F, P]
        lib.oracle_quantize_weights.argtypes = [P, I, I64, I64, F, P, P, P]
        lib.oracle_quantize_acts.argtypes = [P, I, I64, I64, I, I, F, P, P]
        lib.oracle_forward.argtypes = [P, I, P, I, P, P, P, I64, I64, I64, I, P, I, P]
        lib.oracle_forward_at.argtypes = [P, I, P, I, P, P, P, I64, I64, I64, I, I64, P, P, P, I,
                                          P]
        lib.oracle_to_bf16.argtypes = [P, P, I64]
        lib.oracle_rmsnorm.argtypes = [P, P, I64, I64, F, P, P]
        lib.oracle_sumsq.argtypes = [P, I64, P]
        lib.oracle_layernorm.argtypes = [P, P, I64, I64, F, P, P]
        lib.oracle_layernorm_sums.argtypes = [P, I64, P, P]
        lib.oracle_hadamard_block.argtypes = [I64]
        lib.oracle_hadamard_block.restype = I64
        lib.oracle_hadamard_rows.argtypes = [P, I, I64, I64, P]
        lib.oracle_quantize_acts_rotated.argtypes = [P, I, I64, I64, I, I, F, P, P]
        lib.oracle_quantize_weights_rotated.argtypes = [P, I, I64, I64, F, P, P, P]
        lib.oracle_backward.argtypes = [P, P, I, P, I, P, P, P, I, P, I, I64, I64, I64, P, P, P]
        for name in ("oracle_gamma", "oracle_quantize_weights", "oracle_quantize_acts",
                     "oracle_forward", "oracle_forward_at", "oracle_hadamard_rows",
                     "oracle_rmsnorm", "oracle_sumsq", "oracle_layernorm",
                     "oracle_layernorm_sums",
                     "oracle_quantize_acts_rotated", "oracle_quantize_weights_rotated",
                     "oracle_backward"):
            getattr(lib, name).restype = I
        lib.oracle_to_bf16.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st, what):
    if st != 0:
        raise OracleError("%s failed with status %d" % (what, st))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits), got %s" % a.dtype)


def gamma(W: np.ndarray, eps: float = 1e-5) -> np.float32:
    W = np.ascontiguousarray(W)
    N, K = W.shape
    out = np.zeros(1, np.float32)
    _check(_load().oracle_gamma(_ptr(W), _dtype_code(W), N, K, eps, _ptr(out)), "oracle_gamma")
    return out[0]


def quantize_weights(W: np.ndarray, eps: float = 1e-5):
    """Returns (packed uint8 [N, K/4], gamma float32, codes int8 [N, K])."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    packed = np.zeros((N, K // 4), np.uint8)
    g = np.zeros(1, np.float32)
    codes = np.zeros((N, K), np.int8)
    _check(_load().oracle_quantize_weights(_ptr(W), _dtype_code(W), N, K, eps, _ptr(packed),
                                           _ptr(g), _ptr(codes)), "oracle_quantize_weights")
    return packed, g[0], codes


def quantize_acts(X: np.ndarray, bits: int = 8, gran: int = PER_TOKEN, eps: float = 1e-5):
    """Returns (Xq, act_scale).  Xq is int8 [M, K] for bits=8, uint8 [M, K/2] for bits=4."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    if bits == 8:
        Xq = np.zeros((M, K), np.int8)
    else:
        Xq = np.zeros((M, K // 2), np.uint8)
    scale = np.zeros(M if gran == PER_TOKEN else 1, np.float32)
    _check(_load().oracle_quantize_acts(_ptr(X), _dtype_code(X), M, K, bits, gran, eps, _ptr(Xq),
                                        _ptr(scale)), "oracle_quantize_acts")
    return Xq, scale


def _fwd_common(Xq, bits, act_scale, packed, gamma_, bias):
    Xq = np.ascontiguousarray(Xq)
    act_scale = np.ascontiguousarray(act_scale, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    g = np.array([gamma_], np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    M = Xq.shape[0]
    K = Xq.shape[1] * (1 if bits == 8 else 2)
    N = packed.shape[0]
    return Xq, act_scale, packed, g, b, M, N, K


def forward(Xq, bits, act_scale, gran, packed, gamma_, bias=None, epi=EPI_NONE,
            y_dtype=F32):
    """Returns (Y [M, N] float32 or uint16 bf16 bits, acc int32 [M, N])."""
    Xq, act_scale, packed, g, b, M, N, K = _fwd_common(Xq, bits, act_scale, packed, gamma_, bias)
    Y = np.zeros((M, N), np.float32 if y_dtype == F32 else np.uint16)
    acc = np.zeros((M, N), np.int32)
    _check(_load().oracle_forward(_ptr(Xq), bits, _ptr(act_scale), gran, _ptr(packed), _ptr(g),
                                  _ptr(b), M, N, K, epi, _ptr(Y), y_dtype, _ptr(acc)),
           "oracle_forward")
    return Y, acc


def forward_at(Xq, bits, act_scale, gran, packed, gamma_, ms, ns, bias=None, epi=EPI_NONE,
               y_dtype=F32):
    """The outputs at positions (ms[i], ns[i]): returns (y [count], acc int32 [count])."""
    Xq, act_scale, packed, g, b, M, N, K = _fwd_common(Xq, bits, act_scale, packed, gamma_, bias)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    count = ms.shape[0]
    Y = np.zeros(count, np.float32 if y_dtype == F32 else np.uint16)
    acc = np.zeros(count, np.int32)
    _check(_load().oracle_forward_at(_ptr(Xq), bits, _ptr(act_scale), gran, _ptr(packed),
                                     _ptr(g), _ptr(b), M, N, K, epi, count, _ptr(ms), _ptr(ns),
                                     _ptr(Y), y_dtype, _ptr(acc)), "oracle_forward_at")
    return Y, acc


def to_bf16(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.zeros(y.shape, np.uint16)
    _load().oracle_to_bf16(_ptr(y), _ptr(out), y.size)
    return out


def bitlinear(X, packed, gamma_, bits=8, gran=PER_TOKEN, bias=None, epi=EPI_NONE, y_dtype=F32,
              eps=1e-5):
    """The whole layer on pre-packed weights: quantize_acts then forward."""
    Xq, s = quantize_acts(X, bits, gran, eps)
    Y, acc = forward(Xq, bits, s, gran, packed, gamma_, bias, epi, y_dtype)
    return Y, acc, Xq, s


def rmsnorm(X: np.ndarray, delta=None, eps: float = 1e-6):
    """Residual add and RMS norm of bf16 rows (uint16 bit patterns [M, K]):
    returns (x', h) with x' = bf16(x + delta) (or x) and h = bf16(x' / rms(x'))."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M, K = X.shape
    d = None if delta is None else np.ascontiguousarray(delta, dtype=np.uint16)
    x_out = np.empty_like(X)
    h_out = np.empty_like(X)
    _check(_load().oracle_rmsnorm(_ptr(X), None if d is None else _ptr(d), M, K, eps,
                                  _ptr(x_out), _ptr(h_out)), "rmsnorm")
    return x_out, h_out


def layernorm(X: np.ndarray, delta=None, eps: float = 1e-5):
    """Residual add and non-affine layer norm of bf16 rows (uint16 bit patterns [M, K]):
    returns (x', h) with x' = bf16(x + delta) (or x) and h = bf16((x' - mean) / sqrt(var
    + eps)), var the biased variance."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M, K = X.shape
    d = None if delta is None else np.ascontiguousarray(delta, dtype=np.uint16)
    x_out = np.empty_like(X)
    h_out = np.empty_like(X)
    _check(_load().oracle_layernorm(_ptr(X), None if d is None else _ptr(d), M, K, eps,
                                    _ptr(x_out), _ptr(h_out)), "layernorm")
    return x_out, h_out


def layernorm_sums(row: np.ndarray):
    """(fp64(S1), fp64(D)) of one row of bf16 values: S1 the exact sum, D = K S2 - S1^2
    with S2 the exact sum of squares, each rounded once to fp64 (nearest, ties to even).
    The row's mean is S1 / K and its variance D / K^2."""
    row = np.ascontiguousarray(row, dtype=np.uint16).reshape(-1)
    out = np.zeros(2, np.float64)
    _check(_load().oracle_layernorm_sums(_ptr(row), row.size, _ptr(out[0:]), _ptr(out[1:])),
           "layernorm_sums")
    return float(out[0]), float(out[1])


def sumsq(row: np.ndarray) -> float:
    """The sum of squares of one row of bf16 values (uint16 bit patterns), exact, rounded
    once to fp64 (nearest, ties to even): the S of the RMS norm."""
    row = np.ascontiguousarray(row, dtype=np.uint16).reshape(-1)
    out = np.zeros(1, np.float64)
    _check(_load().oracle_sumsq(_ptr(row), row.size, _ptr(out)), "sumsq")
    return float(out[0])


def hadamard_block(K: int) -> int:
    """Block size b of the rotation on a K-wide axis: the largest power of two dividing
    K, at most 8192."""
    return int(_load().oracle_hadamard_block(K))


def hadamard_rows(X: np.ndarray) -> np.ndarray:
    """Rows of X (float32, or uint16 bf16 bits) times the block-diagonal unnormalized
    Hadamard matrix, in fp32 by the fast transform (stage h = 1, 2, ..., b/2)."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    Y = np.zeros((M, K), np.float32)
    _check(_load().oracle_hadamard_rows(_ptr(X), _dtype_code(X), M, K, _ptr(Y)),
           "oracle_hadamard_rows")
    return Y


def quantize_acts_rotated(X: np.ndarray, bits: int = 4, gran: int = PER_TOKEN, eps: float = 1e-5):
    """quantize_acts of hadamard_rows(X): returns (Xq, act_scale)."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    Xq = np.zeros((M, K) if bits == 8 else (M, K // 2), np.int8 if bits == 8 else np.uint8)
    scale = np.zeros(M if gran == PER_TOKEN else 1, np.float32)
    _check(_load().oracle_quantize_acts_rotated(_ptr(X), _dtype_code(X), M, K, bits, gran, eps,
                                                _ptr(Xq), _ptr(scale)),
           "oracle_quantize_acts_rotated")
    return Xq, scale


def quantize_weights_rotated(W: np.ndarray, eps: float = 1e-5):
    """quantize_weights of hadamard_rows(W), gamma divided by the block size b: returns
    (packed uint8 [N, K/4], gamma float32, codes int8 [N, K])."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    packed = np.zeros((N, K // 4), np.uint8)
    g = np.zeros(1, np.float32)
    codes = np.zeros((N, K), np.int8)
    _check(_load().oracle_quantize_weights_rotated(_ptr(W), _dtype_code(W), N, K, eps,
                                                   _ptr(packed), _ptr(g), _ptr(codes)),
           "oracle_quantize_weights_rotated")
    return packed, g[0], codes


def backward(dY: np.ndarray, Xq: np.ndarray, bits: int, act_scale, gran: int, packed: np.ndarray,
             gamma_, X=None, W=None, want=("dX", "dW", "dbias")):
    """dY uint16 bf16 bits [M, N]; Xq, act_scale, packed, gamma as the forward takes them;
    X, W (float32 or bf16 bits) only for the int4 masks.  Returns a dict of float64 arrays."""
    dY = np.ascontiguousarray(dY, dtype=np.uint16)
    Xq = np.ascontiguousarray(Xq)
    act_scale = np.ascontiguousarray(act_scale, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    g = np.array([gamma_], np.float32)
    M, N = dY.shape
    K = packed.shape[1] * 4
    out = {}
    dX = np.zeros((M, K), np.float64) if "dX" in want else None
    dW = np.zeros((N, K), np.float64) if "dW" in want else None
    db = np.zeros(N, np.float64) if "dbias" in want else None
    X = None if X is None else np.ascontiguousarray(X)
    W = None if W is None else np.ascontiguousarray(W)
    _check(_load().oracle_backward(_ptr(dY), _ptr(Xq), bits, _ptr(act_scale), gran, _ptr(packed),
                                   _ptr(g), _ptr(X), 0 if X is None else _dtype_code(X),
                                   _ptr(W), 0 if W is None else _dtype_code(W), M, N, K,
                                   _ptr(dX), _ptr(dW), _ptr(db)), "oracle_backward")
    for name, a in (("dX", dX), ("dW", dW), ("dbias", db)):
        if a is not None:
            out[name] = a
    return out
