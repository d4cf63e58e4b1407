"""The no-allocation entry point (bitlinear_forward_fused_noalloc) against the entry
point whose kernels it shares (bitlinear_forward_fused with a caller workspace): the
same results to the bit, on two calls in a row with the second one smaller, so that
the second call runs on scratch that still holds the first call's contents."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, say, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (M, K, N, bits, gran, epilogue, out dtype, x scale) of the first and second call; the
# second is smaller in M (and here and there in K, N), and per-tensor cases shrink the
# input's magnitude so that a stale absmax left in scratch would change every code.
CASES = [
    ("prefill int8", (2048, 2560, 6912, 8, "token", "relu2", torch.bfloat16, 1.0),
     (300, 2560, 512, 8, "token", "relu2", torch.bfloat16, 1.0)),
    ("prefill int4 (FP6 x FP4)", (1024, 2560, 768, 4, "token", None, torch.float32, 1.0),
     (256, 2560, 384, 4, "token", None, torch.float32, 1.0)),
    ("per tensor int8", (700, 1024, 640, 8, "tensor", None, torch.float32, 8.0),
     (130, 1024, 640, 8, "tensor", None, torch.float32, 0.25)),
    ("per tensor int4", (512, 512, 256, 4, "tensor", "relu2", torch.bfloat16, 8.0),
     (200, 512, 256, 4, "tensor", "relu2", torch.bfloat16, 0.25)),
    ("decode 16 tokens then 1", (16, 6912, 2560, 8, "token", None, torch.bfloat16, 1.0),
     (1, 6912, 2560, 8, "token", None, torch.bfloat16, 1.0)),
    ("small int8 GEMM", (40, 256, 130, 8, "token", None, torch.int32, 1.0),
     (9, 128, 64, 8, "token", None, torch.int32, 1.0)),
]


def _inputs(M, K, N, scale, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    X = (scale * torch.randn((M, K), device=DEV, generator=g)).to(torch.bfloat16)
    W = 0.02 * torch.randn((N, K), device=DEV, generator=g)
    packed, gamma = bl.quantize_weights(W)
    return X, packed, gamma


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry(name, first, second):
    for i, (M, K, N, bits, gran, epi, odt, scale) in enumerate((first, second)):
        say("noalloc", name, "call", i + 1, dict(M=M, K=K, N=N, bits=bits, gran=gran))
        X, packed, gamma = _inputs(M, K, N, scale, 100 + i)
        y_ref = torch.empty((M, N), dtype=odt, device=DEV)
        bl.forward_fused(X, packed, gamma, bits=bits, gran=gran, epilogue=epi, out=y_ref)
        y = torch.full((M, N), 7, dtype=odt, device=DEV)
        bl.forward_fused_noalloc(X, packed, gamma, y, bits=bits, gran=gran, epilogue=epi)
        torch.cuda.synchronize()
        assert_same_bytes(to_host(y), to_host(y_ref), "%s call %d" % (name, i + 1))


def test_noalloc_rejects_oversized_call_before_launch():
    X = torch.empty((16, 16), dtype=torch.bfloat16, device=DEV)
    packed = torch.empty((16, 4), dtype=torch.uint8, device=DEV)
    gamma = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.empty((16, 16), dtype=torch.float32, device=DEV)
    # the shapes passed claim far more tokens than the scratch can hold: rejected on the
    # host, so the small tensors are never read past their ends
    L = bl.lib()
    st = L.bitlinear_forward_fused_noalloc(X.data_ptr(), bl.BL_BF16, 8, bl.BL_PER_TOKEN, 1e-5,
                                           packed.data_ptr(), gamma.data_ptr(), None, 8192,
                                           28672, 8192, bl.BL_EPI_NONE, y.data_ptr(), bl.BL_F32,
                                           None)
    assert st == bl.BL_EWORKSPACE
    assert "scratch" in L.bitlinear_last_error().decode()
    assert np.isfinite(to_host(gamma)).all()
