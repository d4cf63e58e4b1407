"""The Python binding checks every tensor before the C call (dtype, shape, layout,
device), so a misused tensor raises BitLinearError instead of reaching a kernel as an
out-of-bounds or host address.  No GPU: the tensors here are CPU or meta tensors, which
every check must reject before any pointer is handed to the library."""
from __future__ import annotations

import pytest
import torch

import ternary_weight_quantized_bitlinear_amd as bl

E = bl.BitLinearError
M, K, N = 8, 256, 512


def t(shape, dtype=torch.float32, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


def _status(fn):
    with pytest.raises(E) as ei:
        fn()
    return ei.value.status, str(ei.value)


def test_library_present():
    bl.lib()


CASES = [
    # forward on quantized activations
    ("forward: float codes", lambda: bl.forward(t((M, K)), t((M,)), t((N, K // 4), torch.uint8),
                                                t((1,))), bl.BL_EINVAL, "dtype"),
    ("forward: packed too narrow", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                                      t((N, K // 8), torch.uint8), t((1,))),
     bl.BL_ESHAPE, "packed"),
    ("forward: int8-wide codes as int4", lambda: bl.forward(t((M, K), torch.uint8), t((M,)),
                                                            t((N, K // 4), torch.uint8), t((1,)),
                                                            bits=4),
     bl.BL_ESHAPE, "packed"),
    ("forward: scale length", lambda: bl.forward(t((M, K), torch.int8), t((M - 1,)),
                                                 t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_ESHAPE, "act_scale"),
    ("forward: per-tensor scale length", lambda: bl.forward(
        t((M, K), torch.int8), t((M,)), t((N, K // 4), torch.uint8), t((1,)), gran="tensor"),
     bl.BL_ESHAPE, "act_scale"),
    ("forward: gamma length", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                                 t((N, K // 4), torch.uint8), t((2,))),
     bl.BL_ESHAPE, "gamma"),
    ("forward: gamma dtype", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                                t((N, K // 4), torch.uint8), t((1,), torch.float64)),
     bl.BL_EINVAL, "gamma"),
    ("forward: bias length", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                                t((N, K // 4), torch.uint8), t((1,)),
                                                bias=t((N + 1,))), bl.BL_ESHAPE, "bias"),
    ("forward: out shape", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                              t((N, K // 4), torch.uint8), t((1,)),
                                              out=t((M, N - 1))), bl.BL_ESHAPE, "out"),
    ("forward: out dtype", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                              t((N, K // 4), torch.uint8), t((1,)),
                                              out=t((M, N), torch.float16)), bl.BL_EINVAL, "out"),
    ("forward: strided codes", lambda: bl.forward(t((K, M), torch.int8).t(), t((M,)),
                                                  t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_EINVAL, "contiguous"),
    ("forward: host tensors", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                                 t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_EINVAL, "GPU"),
    ("forward: meta tensors", lambda: bl.forward(t((M, K), torch.int8, "meta"),
                                                 t((M,), device="meta"),
                                                 t((N, K // 4), torch.uint8, "meta"),
                                                 t((1,), device="meta")), bl.BL_EINVAL, "GPU"),
    ("forward: bits", lambda: bl.forward(t((M, K), torch.int8), t((M,)),
                                         t((N, K // 4), torch.uint8), t((1,)), bits=6),
     bl.BL_EINVAL, "bits"),
    ("forward: 1-D codes", lambda: bl.forward(t((K,), torch.int8), t((M,)),
                                              t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_ESHAPE, "Xq"),
    # fused
    ("fused: int codes as X", lambda: bl.forward_fused(t((M, K), torch.int8),
                                                       t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_EINVAL, "X"),
    ("fused: packed K mismatch", lambda: bl.forward_fused(t((M, K)), t((N, K // 4 + 4), torch.uint8),
                                                          t((1,))), bl.BL_ESHAPE, "packed"),
    ("fused: 3-D X", lambda: bl.forward_fused(t((1, M, K)), t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_ESHAPE, "X"),
    ("fused: workspace dtype", lambda: bl.forward_fused(
        t((2048, K)), t((N, K // 4), torch.uint8), t((1,)), workspace=t((1 << 20,))),
     bl.BL_EINVAL, "GPU"),
    ("noalloc: out shape", lambda: bl.forward_fused_noalloc(
        t((M, K)), t((N, K // 4), torch.uint8), t((1,)), t((M, N + 1))), bl.BL_ESHAPE, "out"),
    ("noalloc: host tensors", lambda: bl.forward_fused_noalloc(
        t((M, K)), t((N, K // 4), torch.uint8), t((1,)), t((M, N))), bl.BL_EINVAL, "GPU"),
    # batched and multi-part
    ("batched: gamma per problem", lambda: bl.forward_fused_batched(
        t((4, 1, K)), t((4, N, K // 4), torch.uint8), t((3,))), bl.BL_ESHAPE, "gamma"),
    ("batched: packed problems", lambda: bl.forward_fused_batched(
        t((4, 1, K)), t((5, N, K // 4), torch.uint8), t((4,))), bl.BL_ESHAPE, "packed"),
    ("batched: bias", lambda: bl.forward_fused_batched(
        t((4, 1, K)), t((4, N, K // 4), torch.uint8), t((4,)), bias=t((N,))), bl.BL_ESHAPE, "bias"),
    ("multi: gamma per part", lambda: bl.forward_multi(
        t((M, K), torch.int8), t((M,)), t((3, N, K // 4), torch.uint8), t((1,))),
     bl.BL_ESHAPE, "gamma"),
    ("multi: out parts", lambda: bl.forward_multi(
        t((M, K), torch.int8), t((M,)), t((3, N, K // 4), torch.uint8), t((3,)),
        out=t((2, M, N))), bl.BL_ESHAPE, "out"),
    # quantizers
    ("quantize_weights: 1-D W", lambda: bl.quantize_weights(t((K,))), bl.BL_ESHAPE, "W"),
    ("quantize_weights: out packed", lambda: bl.quantize_weights(
        t((N, K)), out=(t((N, K // 2), torch.uint8), t((1,)))), bl.BL_ESHAPE, "packed"),
    ("quantize_weights: int W", lambda: bl.quantize_weights(t((N, K), torch.int8)),
     bl.BL_EINVAL, "W"),
    ("quantize_weights_rotated: out gamma", lambda: bl.quantize_weights_rotated(
        t((N, K)), out=(t((N, K // 4), torch.uint8), t((2,)))), bl.BL_ESHAPE, "gamma"),
    ("quantize_acts: int4 out width", lambda: bl.quantize_acts(
        t((M, K)), bits=4, out=(t((M, K), torch.int8), t((M,)))), bl.BL_ESHAPE, "Xq"),
    ("quantize_acts: out scale", lambda: bl.quantize_acts(
        t((M, K)), gran="tensor", out=(t((M, K), torch.int8), t((M,)))), bl.BL_ESHAPE, "act_scale"),
    ("quantize_acts_rotated: host X", lambda: bl.quantize_acts_rotated(t((M, K))),
     bl.BL_EINVAL, "GPU"),
    # glue
    ("rmsnorm: fp32 X", lambda: bl.rmsnorm(t((M, K))), bl.BL_EINVAL, "X"),
    ("rmsnorm: delta shape", lambda: bl.rmsnorm(t((M, K), torch.bfloat16),
                                                t((M, K - 8), torch.bfloat16)), bl.BL_ESHAPE, "delta"),
    ("rmsnorm: out shape", lambda: bl.rmsnorm(t((M, K), torch.bfloat16),
                                              out=t((M, K + 8), torch.bfloat16)), bl.BL_ESHAPE, "out"),
    ("rmsnorm_quantize: out codes", lambda: bl.rmsnorm_quantize(
        t((M, K), torch.bfloat16), out=(t((M, K), torch.bfloat16), t((M, K // 2), torch.int8),
                                        t((M,)))), bl.BL_ESHAPE, "Xq"),
    ("layernorm: fp32 X", lambda: bl.layernorm(t((M, K))), bl.BL_EINVAL, "X"),
    ("layernorm: delta dtype", lambda: bl.layernorm(t((M, K), torch.bfloat16), t((M, K))),
     bl.BL_EINVAL, "delta"),
    ("layernorm: host tensors", lambda: bl.layernorm(t((M, K), torch.bfloat16)),
     bl.BL_EINVAL, "GPU"),
    ("layernorm_quantize: out scale", lambda: bl.layernorm_quantize(
        t((M, K), torch.bfloat16), out=(t((M, K), torch.bfloat16), t((M, K), torch.int8),
                                        t((M + 1,)))), bl.BL_ESHAPE, "act_scale"),
    ("layernorm_quantize: bits", lambda: bl.layernorm_quantize(t((M, K), torch.bfloat16), bits=2),
     bl.BL_EINVAL, "bits"),
    ("norm_forward: delta without x_out", lambda: bl.norm_forward(
        t((M, K), torch.bfloat16), t((N, K // 4), torch.uint8), t((1,)),
        delta=t((M, K), torch.bfloat16)), bl.BL_EINVAL, "x_out"),
    ("norm_forward: bad norm", lambda: bl.norm_forward(
        t((M, K), torch.bfloat16), t((N, K // 4), torch.uint8), t((1,)), norm="l2"),
     bl.BL_EINVAL, "norm"),
    ("norm_forward: parts gamma", lambda: bl.norm_forward(
        t((M, K), torch.bfloat16), t((3, N, K // 4), torch.uint8), t((1,))), bl.BL_ESHAPE, "gamma"),
    ("norm_forward: x_out shape", lambda: bl.norm_forward(
        t((M, K), torch.bfloat16), t((N, K // 4), torch.uint8), t((1,)),
        delta=t((M, K), torch.bfloat16), x_out=t((M, K + 16), torch.bfloat16)), bl.BL_ESHAPE, "x_out"),
    ("norm_forward: host tensors", lambda: bl.norm_forward(
        t((M, K), torch.bfloat16), t((N, K // 4), torch.uint8), t((1,))), bl.BL_EINVAL, "GPU"),
    # backward
    ("backward: fp32 dY", lambda: bl.backward(t((M, N)), t((M, K), torch.int8), t((M,)),
                                              t((N, K // 4), torch.uint8), t((1,))),
     bl.BL_EINVAL, "dY"),
    ("backward: codes shape", lambda: bl.backward(
        t((M, N), torch.bfloat16), t((M, K // 2), torch.int8), t((M,)),
        t((N, K // 4), torch.uint8), t((1,))), bl.BL_ESHAPE, "Xq"),
    ("backward: packed rows", lambda: bl.backward(
        t((M, N), torch.bfloat16), t((M, K), torch.int8), t((M,)),
        t((N + 1, K // 4), torch.uint8), t((1,))), bl.BL_ESHAPE, "packed"),
    ("backward: mask input shape", lambda: bl.backward(
        t((M, N), torch.bfloat16), t((M, K // 2), torch.uint8), t((M,)),
        t((N, K // 4), torch.uint8), t((1,)), bits=4, X=t((M, K + 16))), bl.BL_ESHAPE, "X"),
    ("backward: dX out", lambda: bl.backward(
        t((M, N), torch.bfloat16), t((M, K), torch.int8), t((M,)),
        t((N, K // 4), torch.uint8), t((1,)), want=("dX",), out={"dX": t((M, K - 1))}),
     bl.BL_ESHAPE, "dX"),
    ("backward: host tensors", lambda: bl.backward(
        t((M, N), torch.bfloat16), t((M, K), torch.int8), t((M,)),
        t((N, K // 4), torch.uint8), t((1,))), bl.BL_EINVAL, "GPU"),
]


@pytest.mark.parametrize("name,call,status,word", CASES, ids=[c[0] for c in CASES])
def test_binding_rejects(name, call, status, word):
    st, msg = _status(call)
    assert st == status, msg
    assert word in msg, msg
