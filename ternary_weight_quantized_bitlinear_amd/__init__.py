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
* :func:`forward_fused_noalloc` -> ``bitlinear_forward_fused_noalloc`` (no workspace)
* :func:`forward_multi`     -> ``bitlinear_forward_multi`` (several projections of one input)
* :func:`rmsnorm`           -> ``bitlinear_rmsnorm`` (glue between layers)
* :func:`rmsnorm_quantize`  -> ``bitlinear_rmsnorm_quantize`` (glue + next layer's quantizer)
* :func:`layernorm`         -> ``bitlinear_layernorm`` (the same glue, non-affine layer norm)
* :func:`layernorm_quantize` -> ``bitlinear_layernorm_quantize``
* :func:`norm_forward`      -> ``bitlinear_norm_forward`` (residual + norm + quantize + projections)
* :func:`backward`          -> ``bitlinear_backward`` (straight-through-estimator gradients)
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# BITLINEAR_LIB selects another build of the library (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("BITLINEAR_LIB") or os.path.join(PKG_DIR, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "bitlinear.h")

# enums of include/bitlinear.h
BL_OK, BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EUNSUPPORTED, BL_EDEVICE, BL_EWORKSPACE = range(7)
BL_F32, BL_BF16, BL_I32 = 0, 1, 2
BL_PER_TOKEN, BL_PER_TENSOR = 0, 1
BL_EPI_NONE, BL_EPI_RELU2 = 0, 1
(BL_OP_QUANTIZE_WEIGHTS, BL_OP_QUANTIZE_ACTS, BL_OP_FORWARD, BL_OP_FORWARD_FUSED,
 BL_OP_BACKWARD, BL_OP_NORM_FORWARD) = range(6)
BL_NORM_NONE, BL_NORM_RMS, BL_NORM_LAYER = range(3)


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
        L.bitlinear_forward_fused_noalloc.argtypes = [P, I, I, I, F, P, P, P, I64, I64, I64, I,
                                                      P, I, P]
        L.bitlinear_noalloc_scratch_bytes.argtypes = []
        L.bitlinear_noalloc_scratch_bytes.restype = SZ
        L.bitlinear_rmsnorm.argtypes = [P, P, P, I64, I64, F, P]
        L.bitlinear_rmsnorm_quantize.argtypes = [P, P, P, I64, I64, F, I, I, F, P, P, P, SZ, P]
        L.bitlinear_layernorm.argtypes = [P, P, P, I64, I64, F, P]
        L.bitlinear_layernorm_quantize.argtypes = [P, P, P, I64, I64, F, I, I, F, P, P, P, SZ, P]
        L.bitlinear_norm_forward.argtypes = [P, P, P, I, F, I, I, F, P, P, P, I64, I64, I64, I64, I,
                                             P, I, P, SZ, P]
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
                  "bitlinear_forward_multi", "bitlinear_forward_fused_noalloc",
                  "bitlinear_rmsnorm", "bitlinear_rmsnorm_quantize", "bitlinear_layernorm",
                  "bitlinear_layernorm_quantize", "bitlinear_norm_forward",
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
        _arg(workspace, "workspace", None, (torch.uint8,))
        if workspace.device != device:
            _fail(BL_EINVAL, "workspace is on %s, the operands on %s" % (workspace.device, device))
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def workspace_size(op: int, M: int, N: int, K: int, bits: int = 8, gran="token") -> int:
    return lib().bitlinear_workspace_size(op, M, N, K, bits, _gran_code(gran))


# ------------------------------------------------------------------ argument checks
# Every tensor is checked before the C call: the C ABI sees only pointers and sizes, so a
# tensor of the wrong shape, dtype or device, or a strided view, would otherwise reach the
# kernels as an out-of-bounds or host address.  Order: dtype, shape, layout, device.

def _fail(status, msg):
    raise BitLinearError(status, msg)


def _dims(t, name, ndim):
    if t is None:
        _fail(BL_EINVAL, "%s is required" % name)
    if t.dim() != ndim:
        _fail(BL_ESHAPE, "%s must have %d dimensions, has shape %s" % (name, ndim, tuple(t.shape)))
    return tuple(t.shape)


def _arg(t, name, shape, dtypes, optional=False):
    if t is None:
        if optional:
            return
        _fail(BL_EINVAL, "%s is required" % name)
    if dtypes is not None and t.dtype not in dtypes:
        _fail(BL_EINVAL, "%s has dtype %s, expected %s" % (
            name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if shape is not None and tuple(t.shape) != tuple(shape):
        _fail(BL_ESHAPE, "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        _fail(BL_EINVAL, "%s must be contiguous" % name)


def _gpu(**tensors):
    """All given tensors (None skipped) on one GPU: returns that device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            _fail(BL_EINVAL, "%s must be a GPU tensor (is on %s)" % (name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            _fail(BL_EINVAL, "%s is on %s, the other operands on %s" % (name, t.device, dev))
    return dev


def _bits(bits):
    if bits not in (8, 4):
        _fail(BL_EINVAL, "bits must be 8 or 4")
    return bits


def _float_types():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def _code_types():
    torch = _torch()
    return (torch.int8, torch.uint8)


def _out_types():
    torch = _torch()
    return (torch.float32, torch.bfloat16, torch.int32)


def _code_cols(K, bits):
    """Bytes per row of the activation codes: K (int8) or K/2 (two int4 per byte)."""
    return K if bits == 8 else K // 2


def _scale_len(M, g):
    return M if g == BL_PER_TOKEN else 1


# ------------------------------------------------------------------ entry points
# Each entry point: dimensions, then every tensor's dtype, shape and layout, then one
# device for all of them; only then are outputs allocated and the library called.

def quantize_weights(W, eps: float = 1e-5, workspace=None, stream=None, out=None):
    """W [N, K] fp32/bf16 (device) -> (packed uint8 [N, K/4], gamma fp32 [1])."""
    return _quantize_weights(lib().bitlinear_quantize_weights, W, eps, workspace, stream, out)


def quantize_weights_rotated(W, eps: float = 1e-5, workspace=None, stream=None, out=None):
    """quantize_weights of W H (block Hadamard rotation of the rows), gamma divided by the
    block size: use with activations from quantize_acts_rotated."""
    return _quantize_weights(lib().bitlinear_quantize_weights_rotated, W, eps, workspace, stream,
                             out)


def _quantize_weights(fn, W, eps, workspace, stream, out):
    torch = _torch()
    N, K = _dims(W, "W", 2)
    _arg(W, "W", None, _float_types())
    packed, gamma = out if out else (None, None)
    if out:
        _arg(packed, "packed", (N, K // 4), (torch.uint8,))
        _arg(gamma, "gamma", (1,), (torch.float32,))
    dev = _gpu(W=W, packed=packed, gamma=gamma)
    if not out:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_WEIGHTS, 1, N, K), dev, workspace)
    _check(fn(_ptr(W), _dtype_code(W), N, K, eps, _ptr(packed), _ptr(gamma), _ptr(ws), wsb,
              _stream(dev, stream)))
    return packed, gamma


def quantize_acts(X, bits: int = 8, gran="token", eps: float = 1e-5, workspace=None,
                  stream=None, out=None):
    """X [M, K] fp32/bf16 -> (Xq int8 [M, K] or uint8 [M, K/2], act_scale fp32 [M] or [1])."""
    return _quantize_acts(lib().bitlinear_quantize_acts, X, bits, gran, eps, workspace, stream,
                          out)


def quantize_acts_rotated(X, bits: int = 4, gran="token", eps: float = 1e-5, workspace=None,
                          stream=None, out=None):
    """quantize_acts of X H (block Hadamard rotation of the rows)."""
    return _quantize_acts(lib().bitlinear_quantize_acts_rotated, X, bits, gran, eps, workspace,
                          stream, out)


def _quantize_acts(fn, X, bits, gran, eps, workspace, stream, out):
    torch = _torch()
    M, K = _dims(X, "X", 2)
    _arg(X, "X", None, _float_types())
    bits = _bits(bits)
    g = _gran_code(gran)
    Xq, scale = out if out else (None, None)
    if out:
        _arg(Xq, "Xq", (M, _code_cols(K, bits)), _code_types())
        _arg(scale, "act_scale", (_scale_len(M, g),), (torch.float32,))
    dev = _gpu(X=X, Xq=Xq, act_scale=scale)
    if not out:
        Xq = torch.empty((M, _code_cols(K, bits)),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
        scale = torch.empty(_scale_len(M, g), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_ACTS, M, 1, K, bits, g), dev, workspace)
    _check(fn(_ptr(X), _dtype_code(X), M, K, bits, g, eps, _ptr(Xq), _ptr(scale), _ptr(ws), wsb,
              _stream(dev, stream)))
    return Xq, scale


def hadamard_block(K: int) -> int:
    """Block size b of the Hadamard rotation on a K-wide axis."""
    return int(lib().bitlinear_hadamard_block(K))


def _out_arg(out, shape):
    if out is not None:
        _arg(out, "out", shape, _out_types())


def _new_out(out, shape, out_dtype, dev):
    torch = _torch()
    return out if out is not None else torch.empty(shape, dtype=out_dtype or torch.float32,
                                                   device=dev)


def forward(Xq, act_scale, packed, gamma, bits: int = 8, gran="token", bias=None,
            epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """Quantized activations -> Y [M, N] (fp32, bf16 or int32 accumulators)."""
    torch = _torch()
    bits = _bits(bits)
    M, cols = _dims(Xq, "Xq", 2)
    N, _ = _dims(packed, "packed", 2)
    K = cols * (1 if bits == 8 else 2)
    g = _gran_code(gran)
    _arg(Xq, "Xq", None, _code_types())
    _arg(packed, "packed", (N, K // 4), (torch.uint8,))
    _arg(act_scale, "act_scale", (_scale_len(M, g),), (torch.float32,))
    _arg(gamma, "gamma", (1,), (torch.float32,))
    _arg(bias, "bias", (N,), (torch.float32,), optional=True)
    _out_arg(out, (M, N))
    dev = _gpu(Xq=Xq, packed=packed, act_scale=act_scale, gamma=gamma, bias=bias, out=out)
    out = _new_out(out, (M, N), out_dtype, dev)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_forward(_ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma),
                                   _ptr(bias), M, N, K, _epi_code(epilogue), _ptr(out),
                                   _dtype_code(out), _ptr(ws), wsb, _stream(dev, stream)))
    return out


def _fused_args(X, packed, gamma, bias, out):
    torch = _torch()
    M, K = _dims(X, "X", 2)
    N, _ = _dims(packed, "packed", 2)
    _arg(X, "X", None, _float_types())
    _arg(packed, "packed", (N, K // 4), (torch.uint8,))
    _arg(gamma, "gamma", (1,), (torch.float32,))
    _arg(bias, "bias", (N,), (torch.float32,), optional=True)
    _out_arg(out, (M, N))
    dev = _gpu(X=X, packed=packed, gamma=gamma, bias=bias, out=out)
    return M, N, K, dev


def forward_fused(X, packed, gamma, bits: int = 8, gran="token", eps: float = 1e-5, bias=None,
                  epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """Unquantized activations X [M, K] fp32/bf16 -> Y [M, N]: quantize_acts + forward."""
    bits = _bits(bits)
    M, N, K, dev = _fused_args(X, packed, gamma, bias, out)
    g = _gran_code(gran)
    out = _new_out(out, (M, N), out_dtype, dev)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD_FUSED, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_forward_fused(_ptr(X), _dtype_code(X), bits, g, eps, _ptr(packed),
                                         _ptr(gamma), _ptr(bias), M, N, K, _epi_code(epilogue),
                                         _ptr(out), _dtype_code(out), _ptr(ws), wsb,
                                         _stream(dev, stream)))
    return out


def forward_fused_noalloc(X, packed, gamma, out, bits: int = 8, gran="token", eps: float = 1e-5,
                          bias=None, epilogue=None, stream=None):
    """forward_fused without a workspace: the library's fixed per-GPU scratch is used and
    nothing is allocated (`out`, the [M, N] result, must be given)."""
    bits = _bits(bits)
    if out is None:
        _fail(BL_EINVAL, "out is required")
    M, N, K, dev = _fused_args(X, packed, gamma, bias, out)
    _check(lib().bitlinear_forward_fused_noalloc(_ptr(X), _dtype_code(X), bits, _gran_code(gran),
                                                 eps, _ptr(packed), _ptr(gamma), _ptr(bias), M,
                                                 N, K, _epi_code(epilogue), _ptr(out),
                                                 _dtype_code(out), _stream(dev, stream)))
    return out


def forward_fused_batched(X, packed, gamma, bits: int = 8, gran="token", eps: float = 1e-5,
                          bias=None, epilogue=None, out_dtype=None, workspace=None, stream=None,
                          out=None):
    """`batch` independent layers of one shape: X [B, M, K], packed [B, N, K/4], gamma [B],
    bias [B, N] or None -> Y [B, M, N]; problem b is forward_fused(X[b], packed[b], ...)."""
    torch = _torch()
    bits = _bits(bits)
    B, M, K = _dims(X, "X", 3)
    _, N, _ = _dims(packed, "packed", 3)
    _arg(X, "X", None, _float_types())
    _arg(packed, "packed", (B, N, K // 4), (torch.uint8,))
    _arg(gamma, "gamma", (B,), (torch.float32,))
    _arg(bias, "bias", (B, N), (torch.float32,), optional=True)
    _out_arg(out, (B, M, N))
    dev = _gpu(X=X, packed=packed, gamma=gamma, bias=bias, out=out)
    g = _gran_code(gran)
    out = _new_out(out, (B, M, N), out_dtype, dev)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD_FUSED, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_forward_fused_batched(
        _ptr(X), _dtype_code(X), bits, g, eps, _ptr(packed), _ptr(gamma), _ptr(bias), B, M, N, K,
        _epi_code(epilogue), _ptr(out), _dtype_code(out), _ptr(ws), wsb, _stream(dev, stream)))
    return out


def forward_multi(Xq, act_scale, packed, gamma, bits: int = 8, gran="token", bias=None,
                  epilogue=None, out_dtype=None, workspace=None, stream=None, out=None):
    """`parts` projections of one quantized input: Xq [M, K] codes, packed [P, N, K/4],
    gamma [P], bias [P, N] or None -> Y [P, M, N]; part p is forward(Xq, act_scale,
    packed[p], gamma[p:p+1], ...)."""
    torch = _torch()
    bits = _bits(bits)
    M, cols = _dims(Xq, "Xq", 2)
    Pn, N, _ = _dims(packed, "packed", 3)
    K = cols * (1 if bits == 8 else 2)
    g = _gran_code(gran)
    _arg(Xq, "Xq", None, _code_types())
    _arg(packed, "packed", (Pn, N, K // 4), (torch.uint8,))
    _arg(act_scale, "act_scale", (_scale_len(M, g),), (torch.float32,))
    _arg(gamma, "gamma", (Pn,), (torch.float32,))
    _arg(bias, "bias", (Pn, N), (torch.float32,), optional=True)
    _out_arg(out, (Pn, M, N))
    dev = _gpu(Xq=Xq, packed=packed, act_scale=act_scale, gamma=gamma, bias=bias, out=out)
    out = _new_out(out, (Pn, M, N), out_dtype, dev)
    ws, wsb = _workspace(workspace_size(BL_OP_FORWARD, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_forward_multi(
        _ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma), _ptr(bias), Pn, M, N, K,
        _epi_code(epilogue), _ptr(out), _dtype_code(out), _ptr(ws), wsb, _stream(dev, stream)))
    return out


def _norm(entry, X, delta, eps, out, stream):
    torch = _torch()
    M, K = _dims(X, "X", 2)
    _arg(X, "X", None, (torch.bfloat16,))
    _arg(delta, "delta", (M, K), (torch.bfloat16,), optional=True)
    _arg(out, "out", (M, K), (torch.bfloat16,), optional=True)
    dev = _gpu(X=X, delta=delta, out=out)
    if out is None:
        out = torch.empty_like(X)
    _check(entry(_ptr(X), _ptr(delta), _ptr(out), M, K, eps, _stream(dev, stream)))
    return out


def _norm_quantize(entry, X, delta, eps, bits, gran, q_eps, out, workspace, stream):
    torch = _torch()
    bits = _bits(bits)
    M, K = _dims(X, "X", 2)
    g = _gran_code(gran)
    _arg(X, "X", None, (torch.bfloat16,))
    _arg(delta, "delta", (M, K), (torch.bfloat16,), optional=True)
    H, Xq, sc = out if out else (None, None, None)
    if out:
        _arg(H, "H", (M, K), (torch.bfloat16,))
        _arg(Xq, "Xq", (M, _code_cols(K, bits)), _code_types())
        _arg(sc, "act_scale", (_scale_len(M, g),), (torch.float32,))
    dev = _gpu(X=X, delta=delta, H=H, Xq=Xq, act_scale=sc)
    if not out:
        H = torch.empty_like(X)
        Xq = torch.empty((M, _code_cols(K, bits)),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
        sc = torch.empty((_scale_len(M, g),), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace_size(BL_OP_QUANTIZE_ACTS, M, 1, K, bits, g), dev, workspace)
    _check(entry(_ptr(X), _ptr(delta), _ptr(H), M, K, eps, bits, g, q_eps, _ptr(Xq), _ptr(sc),
                 _ptr(ws), wsb, _stream(dev, stream)))
    return H, Xq, sc


def rmsnorm(X, delta=None, eps: float = 1e-6, out=None, stream=None):
    """Residual add and RMS norm of bf16 rows: X [M, K] bf16 (overwritten with X + delta
    when delta is given) -> H [M, K] bf16 = X / rms(X)."""
    return _norm(lib().bitlinear_rmsnorm, X, delta, eps, out, stream)


def rmsnorm_quantize(X, delta=None, eps: float = 1e-6, bits: int = 8, gran="token",
                     q_eps: float = 1e-5, out=None, workspace=None, stream=None):
    """rmsnorm followed by quantize_acts of its output: returns (H, Xq, scale)."""
    return _norm_quantize(lib().bitlinear_rmsnorm_quantize, X, delta, eps, bits, gran, q_eps,
                          out, workspace, stream)


def layernorm(X, delta=None, eps: float = 1e-5, out=None, stream=None):
    """Residual add and non-affine layer norm of bf16 rows: X [M, K] bf16 (overwritten with
    X + delta when delta is given) -> H [M, K] bf16 = (X - mean) / sqrt(var + eps)."""
    return _norm(lib().bitlinear_layernorm, X, delta, eps, out, stream)


def layernorm_quantize(X, delta=None, eps: float = 1e-5, bits: int = 8, gran="token",
                       q_eps: float = 1e-5, out=None, workspace=None, stream=None):
    """layernorm followed by quantize_acts of its output: returns (H, Xq, scale)."""
    return _norm_quantize(lib().bitlinear_layernorm_quantize, X, delta, eps, bits, gran, q_eps,
                          out, workspace, stream)


_NORMS = {None: BL_NORM_NONE, "none": BL_NORM_NONE, "rms": BL_NORM_RMS, "layer": BL_NORM_LAYER}


def norm_forward(X, packed, gamma, delta=None, x_out=None, norm="rms", eps: float = 1e-6,
                 bits: int = 8, gran="token", q_eps: float = 1e-5, bias=None, epilogue=None,
                 out_dtype=None, workspace=None, stream=None, out=None):
    """Residual add, norm, absmax quantization and the projections in one call: X [M, K]
    bf16 (read only), delta [M, K] bf16 or None, x_out [M, K] bf16 (receives X + delta;
    required with delta), packed [N, K/4] or [P, N, K/4], gamma [1] or [P] -> Y [M, N] or
    [P, M, N].  norm: "rms", "layer" or None."""
    torch = _torch()
    bits = _bits(bits)
    if norm not in _NORMS:
        _fail(BL_EINVAL, "norm must be 'rms', 'layer' or None, not %r" % (norm,))
    M, K = _dims(X, "X", 2)
    single = packed is not None and packed.dim() == 2
    if single:
        N, _ = _dims(packed, "packed", 2)
        Pn = 1
    else:
        Pn, N, _ = _dims(packed, "packed", 3)
    g = _gran_code(gran)
    _arg(X, "X", None, (torch.bfloat16,))
    _arg(delta, "delta", (M, K), (torch.bfloat16,), optional=True)
    _arg(x_out, "x_out", (M, K), (torch.bfloat16,), optional=delta is None)
    _arg(packed, "packed", (N, K // 4) if single else (Pn, N, K // 4), (torch.uint8,))
    _arg(gamma, "gamma", (Pn,), (torch.float32,))
    _arg(bias, "bias", (N,) if single else (Pn, N), (torch.float32,), optional=True)
    yshape = (M, N) if single else (Pn, M, N)
    _out_arg(out, yshape)
    dev = _gpu(X=X, delta=delta, x_out=x_out, packed=packed, gamma=gamma, bias=bias, out=out)
    out = _new_out(out, yshape, out_dtype, dev)
    ws, wsb = _workspace(workspace_size(BL_OP_NORM_FORWARD, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_norm_forward(
        _ptr(X), _ptr(delta), _ptr(x_out), _NORMS[norm], eps, bits, g, q_eps, _ptr(packed),
        _ptr(gamma), _ptr(bias), Pn, M, N, K, _epi_code(epilogue), _ptr(out), _dtype_code(out),
        _ptr(ws), wsb, _stream(dev, stream)))
    return out


def backward(dY, Xq, act_scale, packed, gamma, bits: int = 8, gran="token", X=None, W=None,
             want=("dX", "dW", "dbias"), workspace=None, stream=None, out=None):
    """Straight-through-estimator gradients of the layer: dY [M, N] bf16 (the loss's
    gradient with respect to Y) and the forward's Xq, act_scale, packed, gamma -> dict with
    the fp32 gradients requested in `want`: "dX" [M, K], "dW" [N, K], "dbias" [N].  X and
    W (fp32/bf16, 4-bit activations only) switch on the clipping masks.  `out` may hold
    preallocated tensors under the same keys."""
    torch = _torch()
    bits = _bits(bits)
    M, N = _dims(dY, "dY", 2)
    _, kq = _dims(packed, "packed", 2)
    K = kq * 4
    g = _gran_code(gran)
    _arg(dY, "dY", None, (torch.bfloat16,))
    _arg(packed, "packed", (N, kq), (torch.uint8,))
    _arg(Xq, "Xq", (M, _code_cols(K, bits)), _code_types())
    _arg(act_scale, "act_scale", (_scale_len(M, g),), (torch.float32,))
    _arg(gamma, "gamma", (1,), (torch.float32,))
    _arg(X, "X", (M, K), _float_types(), optional=True)
    _arg(W, "W", (N, K), _float_types(), optional=True)
    shapes = {"dX": (M, K), "dW": (N, K), "dbias": (N,)}
    given = {}
    for name in want:
        if name not in shapes:
            raise ValueError("unknown gradient %r" % name)
        t = (out or {}).get(name)
        if t is not None:
            _arg(t, name, shapes[name], (torch.float32,))
        given[name] = t
    dev = _gpu(dY=dY, Xq=Xq, act_scale=act_scale, packed=packed, gamma=gamma, X=X, W=W, **given)
    res = {name: t if t is not None else torch.empty(shapes[name], dtype=torch.float32, device=dev)
           for name, t in given.items()}
    ws, wsb = _workspace(workspace_size(BL_OP_BACKWARD, M, N, K, bits, g), dev, workspace)
    _check(lib().bitlinear_backward(
        _ptr(dY), _ptr(Xq), bits, _ptr(act_scale), g, _ptr(packed), _ptr(gamma), _ptr(X),
        BL_F32 if X is None else _dtype_code(X), _ptr(W), BL_F32 if W is None else _dtype_code(W),
        M, N, K, _ptr(res.get("dX")), _ptr(res.get("dW")), _ptr(res.get("dbias")), _ptr(ws), wsb,
        _stream(dev, stream)))
    return res
