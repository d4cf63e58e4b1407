"""Python binding of the MI355X BitLinear library (libbitlinear.so, C ABI in
include/bitlinear.h).

Argument marshalling only: every step of the BitLinear forward pass runs in the
library's HIP kernels.  torch supplies device memory and the current stream.
There is no CPU fallback: if the library has not been built, importing works
but every call raises :class:`BitLinearError`.

The functions mirror the C entry points:

* :func:`quantize_weights`  -> ``bitlinear_quantize_weights``
* :func:`quantize_acts`     -> ``bitlinear_quantize_acts``
* :func:`forward`           -> ``bitlinear_forward``
* :func:`forward_fused`     -> ``bitlinear_forward_fused``
* :func:`forward_fused_batched` -> ``bitlinear_forward_fused_batched``
* :func:`forward_multi`     -> ``bitlinear_forward_multi`` (several projections of one input)
* :func:`rmsnorm`           -> ``bitlinear_rmsnorm`` (glue between layers)
* :func:`rmsnorm_quantize`  -> ``bitlinear_rmsnorm_quantize`` (glue + next layer's quantizer)
* :func:`backward`          -> ``bitlinear_backward`` (straight-through-estimator gradients)
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "bitlinear.h")

# enums of include/bitlinear.h
BL_OK, BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EUNSUPPORTED, BL_EDEVICE, BL_EWORKSPACE = range(7)
BL_F32, BL_BF16, BL_I32 = 0, 1, 2
BL_PER_TOKEN, BL_PER_TENSOR = 0, 1
BL_EPI_NONE, BL_EPI_RELU2 = 0, 1
(BL_OP_QUANTIZE_WEIGHTS, BL_OP_QUANTIZE_ACTS, BL_OP_FORWARD, BL_OP_FORWARD_FUSED,
 BL_OP_BACKWARD) = range(5)


class BitLinearError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("bitlinear status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises BitLinearError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BitLinearError(BL_EDEVICE, "libbitlinear.so is not built (%s); run "
                                 "__graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
        L.bitlinear_quantize_weights.argtypes = [P, I, I64, I64, F, P, P, P, SZ, P]
        L.bitlinear_quantize_acts.argtypes = [P, I, I64, I64, I, I, F, P, P, P, SZ, P]
        L.bitlinear_forward.argtypes = [P, I, P, I, P, P, P, I64, I64, I64, I, P, I, P, SZ, P]
        L.bitlinear_forward_fused.argtypes = [P, I, I, I, F, P, P, P, I64, I64, I64, I, P, I, P,
                                              SZ, P]
        L.bitlinear_forward_fused_batched.argtypes = [P, I, I, I, F, P, P, P, I64, I64, I64, I64,
                                                      I, P, I, P, SZ, P]
        L.bitlinear_forward_multi.argtypes = [P, I, P, I, P, P, P, I64, I64, I64, I64, I, P, I, P,
                                              SZ, P]
        L.bitlinear_rmsnorm.argtypes = [P, P, P, I64, I64, F, P]
        L.bitlinear_rmsnorm_quantize.argtypes = [P, P, P, I64, I64, F, I, I, F, P, P, P, SZ, P]
        L.bitlinear_quantize_weights_rotated.argtypes = [P, I, I64, I64, F, P, P, P, SZ, P]
        L.bitlinear_quantize_acts_rotated.argtypes = [P, I, I64, I64, I, I, F, P, P, P, SZ, P]
        L.bitlinear_hadamard_block.argtypes = [I64]
        L.bitlinear_backward.argtypes = [P, P, I, P, I, P, P, P, I, P, I, I64, I64, I64, P, P, P,
                                         P, SZ, P]
        L.bitlinear_hadamard_block.restype = I64
        L.bitlinear_workspace_size.argtypes = [I, I64, I64, I64, I, I]
        L.bitlinear_workspace_size.restype = SZ
        L.bitlinear_status_string.argtypes = [I]
        L.bitlinear_status_string.restype = ctypes.c_char_p
        L.bitlinear_last_error.argtypes = []
        L.bitlinear_last_error.restype = ctypes.c_char_p
        L.bitlinear_version.restype = I
        for n in ("bitlinear_quantize_weights", "bitlinear_quantize_acts", "bitlinear_forward",
                  "bitlinear_forward_fused", "bitlinear_forward_fused_batched",
                  "bitlinear_forward_multi", "bitlinear_rmsnorm", "bitlinear_rmsnorm_quantize",
                  "bitlinear_quantize_weights_rotated", "bitlinear_quantize_acts_rotated",
                  "bitlinear_backward"):
            getattr(L, n).restype = I
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/bitlinear.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bitlinear_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != BL_OK:
        L = lib()
        raise BitLinearError(status, "%s: %s" % (L.bitlinear_status_string(status).decode(),
                                                 L.bitlinear_last_error().decode()))


# ------------------------------------------------------------------ torch helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return BL_F32
    if t.dtype == torch.bfloat16:
        return BL_BF16
    if t.dtype == torch.int32:
        return BL_I32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _gran_code(gran) -> int:
    if gran in ("token", BL_PER_TOKEN):
        return BL_PER_TOKEN
    if gran in ("tensor", BL_PER_TENSOR):
        return BL_PER_TENSOR
    raise ValueError("gran must be 'token' or 'tensor'")


def _epi_code(epilogue) -> int:
    if epilogue in (None, "none", BL_EPI_NONE):
        return BL_EPI_NONE
    if epilogue in ("relu2", BL_EPI_RELU2):
        return BL_EPI_RELU2
    raise ValueError("epilogue must be None or 'relu2'")


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def workspace_size(op: int, M: int, N: int, K: int, bits: int = 8, gran="token") -> int:
    return lib().bitlinear_workspace_size(op, M, N, K, bits, _gran_code(gran))


# ------------------------------------------------------------------ entry points

def quantize_weights(W, eps: float = 1e-5, workspace=None, stream=None, out=None):
    """W [N, K] fp32/bf16 (device) -> (packed uint8 [N, K/4], gamma fp32 [1])."""
    torch = _torch()
    N, K = W.shape
    packed = out[0] if out else torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    gamma = out[1] if out else torch.empty(1, dtype=torch.float32, device=W.device)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_WEIGHTS, 1, N, K), W.device, workspace)
    _check(lib().bitlinear_quantize_weights(_ptr(W), _dtype_code(W), N, K, eps, _ptr(packed),
                                            _ptr(gamma), _ptr(ws), wsb,
                                            _stream(W.device, stream)))
    return packed, gamma


def quantize_acts(X, bits: int = 8, gran="token", eps: float = 1e-5, workspace=None,
                  stream=None, out=None):
    """X [M, K] fp32/bf16 -> (Xq int8 [M, K] or uint8 [M, K/2], act_scale fp32 [M] or [1])."""
    torch = _torch()
    M, K = X.shape
    g = _gran_code(gran)
    if out:
        Xq, scale = out
    else:
        Xq = torch.empty((M, K) if bits == 8 else (M, K // 2),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device=X.device)
        scale = torch.empty(M if g == BL_PER_TOKEN else 1, dtype=torch.float32, device=X.device)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_ACTS, M, 1, K, bits, g), X.device,
                         workspace)
    _check(lib().bitlinear_quantize_acts(_ptr(X), _dtype_code(X), M, K, bits, g, eps, _ptr(Xq),
                                         _ptr(scale), _ptr(ws), wsb, _stream(X.device, stream)))
    return Xq, scale


def hadamard_block(K: int) -> int:
    """Block size b of the Hadamard rotation on a K-wide axis."""
    return int(lib().bitlinear_hadamard_block(K))


def quantize_weights_rotated(W, eps: float = 1e-5, workspace=None, stream=None, out=None):
    """quantize_weights of W H (block Hadamard rotation of the rows), gamma divided by the
    block size: use with activations from quantize_acts_rotated."""
    torch = _torch()
    N, K = W.shape
    packed = out[0] if out else torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    gamma = out[1] if out else torch.empty(1, dtype=torch.float32, device=W.device)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_WEIGHTS, 1, N, K), W.device, workspace)
    _check(lib().bitlinear_quantize_weights_rotated(_ptr(W), _dtype_code(W), N, K, eps,
                                                    _ptr(packed), _ptr(gamma), _ptr(ws), wsb,
                                                    _stream(W.device, stream)))
    return packed, gamma


def quantize_acts_rotated(X, bits: int = 4, gran="token", eps: float = 1e-5, workspace=None,
                          stream=None, out=None):
    """quantize_acts of X H (block Hadamard rotation of the rows)."""
    torch = _torch()
    M, K = X.shape
    g = _gran_code(gran)
    if out:
        Xq, scale = out
    else:
        Xq = torch.empty((M, K) if bits == 8 else (M, K // 2),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device=X.device)
        scale = torch.empty(M if g == BL_PER_TOKEN else 1, dtype=torch.float32, device=X.device)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_ACTS, M, 1, K, bits, g), X.device,
                         workspace)
    _check(lib().bitlinear_quantize_acts_rotated(_ptr(X), _dtype_code(X), M, K, bits, g, eps,
                                                 _ptr(Xq), _ptr(scale), _ptr(ws), wsb,
                                                 _stream(X.device, stream)))
    return Xq, scale


def forward(Xq, act_scale, packed, gamma, bits: int = 8, gran="token", bias=None,
            epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """Quantized activations -> Y [M, N] (fp32, bf16 or int32 accumulators)."""
    torch = _torch()
    M = Xq.shape[0]
    K = Xq.shape[1] * (1 if bits == 8 else 2)
    N = packed.shape[0]
    g = _gran_code(gran)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=Xq.device)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD, M, N, K, bits, g), Xq.device, workspace)
    _check(lib().bitlinear_forward(_ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma),
                                   _ptr(bias), M, N, K, _epi_code(epilogue), _ptr(out),
                                   _dtype_code(out), _ptr(ws), wsb, _stream(Xq.device, stream)))
    return out


def forward_fused(X, packed, gamma, bits: int = 8, gran="token", eps: float = 1e-5, bias=None,
                  epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """Unquantized activations X [M, K] fp32/bf16 -> Y [M, N]: quantize_acts + forward."""
    torch = _torch()
    M, K = X.shape
    N = packed.shape[0]
    g = _gran_code(gran)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=X.device)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD_FUSED, M, N, K, bits, g), X.device,
                         workspace)
    _check(lib().bitlinear_forward_fused(_ptr(X), _dtype_code(X), bits, g, eps, _ptr(packed),
                                         _ptr(gamma), _ptr(bias), M, N, K, _epi_code(epilogue),
                                         _ptr(out), _dtype_code(out), _ptr(ws), wsb,
                                         _stream(X.device, stream)))
    return out


def forward_fused_batched(X, packed, gamma, bits: int = 8, gran="token", eps: float = 1e-5,
                          bias=None, epilogue=None, out_dtype=None, workspace=None, stream=None,
                          out=None):
    """`batch` independent layers of one shape: X [B, M, K], packed [B, N, K/4], gamma [B],
    bias [B, N] or None -> Y [B, M, N]; problem b is forward_fused(X[b], packed[b], ...)."""
    torch = _torch()
    B, M, K = X.shape
    N = packed.shape[1]
    g = _gran_code(gran)
    if out is None:
        out = torch.empty((B, M, N), dtype=out_dtype or torch.float32, device=X.device)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD_FUSED, M, N, K, bits, g), X.device,
                         workspace)
    _check(lib().bitlinear_forward_fused_batched(
        _ptr(X), _dtype_code(X), bits, g, eps, _ptr(packed), _ptr(gamma), _ptr(bias), B, M, N, K,
        _epi_code(epilogue), _ptr(out), _dtype_code(out), _ptr(ws), wsb,
        _stream(X.device, stream)))
    return out


def forward_multi(Xq, act_scale, packed, gamma, bits: int = 8, gran="token", bias=None,
                  epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """`parts` projections of one quantized input: Xq [M, K] codes, packed [P, N, K/4],
    gamma [P], bias [P, N] or None -> Y [P, M, N]; part p is forward(Xq, act_scale,
    packed[p], gamma[p:p+1], ...)."""
    torch = _torch()
    M = Xq.shape[0]
    K = Xq.shape[1] * (1 if bits == 8 else 2)
    Pn, N = packed.shape[0], packed.shape[1]
    g = _gran_code(gran)
    if out is None:
        out = torch.empty((Pn, M, N), dtype=out_dtype or torch.float32, device=Xq.device)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD, M, N, K, bits, g), Xq.device, workspace)
    _check(lib().bitlinear_forward_multi(
        _ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma), _ptr(bias), Pn, M, N, K,
        _epi_code(epilogue), _ptr(out), _dtype_code(out), _ptr(ws), wsb, _stream(Xq.device, stream)))
    return out


def rmsnorm(X, delta=None, eps: float = 1e-6, out=None, stream=None):
    """Residual add and RMS norm of bf16 rows: X [M, K] bf16 (overwritten with X + delta
    when delta is given) -> H [M, K] bf16 = X / rms(X)."""
    torch = _torch()
    M, K = X.shape
    if out is None:
        out = torch.empty_like(X)
    _check(lib().bitlinear_rmsnorm(_ptr(X), _ptr(delta), _ptr(out), M, K, eps,
                                   _stream(X.device, stream)))
    return out


def rmsnorm_quantize(X, delta=None, eps: float = 1e-6, bits: int = 8, gran="token",
                     q_eps: float = 1e-5, out=None, workspace=None, stream=None):
    """rmsnorm followed by quantize_acts of its output: returns (H, Xq, scale)."""
    torch = _torch()
    M, K = X.shape
    g = _gran_code(gran)
    if out is None:
        H = torch.empty_like(X)
        Xq = torch.empty((M, K if bits == 8 else K // 2),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device=X.device)
        sc = torch.empty((M if g == BL_PER_TOKEN else 1,), dtype=torch.float32, device=X.device)
    else:
        H, Xq, sc = out
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_ACTS, M, 1, K, bits, g), X.device,
                         workspace)
    _check(lib().bitlinear_rmsnorm_quantize(_ptr(X), _ptr(delta), _ptr(H), M, K, eps, bits, g,
                                            q_eps, _ptr(Xq), _ptr(sc), _ptr(ws), wsb,
                                            _stream(X.device, stream)))
    return H, Xq, sc


def backward(dY, Xq, act_scale, packed, gamma, bits: int = 8, gran="token", X=None, W=None,
             want=("dX", "dW", "dbias"), workspace=None, stream=None, out=None):
    """Straight-through-estimator gradients of the layer: dY [M, N] bf16 (the loss's
    gradient with respect to Y) and the forward's Xq, act_scale, packed, gamma -> dict with
    the fp32 gradients requested in `want`: "dX" [M, K], "dW" [N, K], "dbias" [N].  X and
    W (fp32/bf16, 4-bit activations only) switch on the clipping masks.  `out` may hold
    preallocated tensors under the same keys."""
    torch = _torch()
    M, N = dY.shape
    K = packed.shape[1] * 4
    g = _gran_code(gran)
    dev = dY.device
    shapes = {"dX": (M, K), "dW": (N, K), "dbias": (N,)}
    res = {}
    for name in want:
        if name not in shapes:
            raise ValueError("unknown gradient %r" % name)
        t = (out or {}).get(name)
        res[name] = t if t is not None else torch.empty(shapes[name], dtype=torch.float32,
                                                        device=dev)
    ws, wsb = _workspace(workspace_size(BL_OP_BACKWARD, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_backward(
        _ptr(dY), _ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma), _ptr(X),
        BL_F32 if X is None else _dtype_code(X), _ptr(W), BL_F32 if W is None else _dtype_code(W),
        M, N, K, _ptr(res.get("dX")), _ptr(res.get("dW")), _ptr(res.get("dbias")), _ptr(ws), wsb,
        _stream(dev, stream)))
    return res
