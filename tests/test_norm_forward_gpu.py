"""GPU parity of bitlinear_norm_forward (residual add + norm + absmax quantization + the
projections of one input; "BitNet 2B4T Guide", "3. Sub-Layer Normalization (SubLN)" and
its block listing; "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
"Implementation", Step 2) and of the decode GEMV's row prologue (one wave quantizes one
token row), which both bitlinear_norm_forward without a norm and bitlinear_forward_fused
at 5..16 bf16 tokens take.
The oracle runs the same steps as separate calls from the same inputs; x' is compared bit
for bit, and every part's Y against the oracle's forward of its own codes (bf16 and int32
outputs bit for bit; fp32 within the path's 1e-5 bar, then bit for bit)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, assert_y_matches, say, to_dev, to_host

pytestmark = pytest.mark.gpu

YDT = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16),
       "i32": (torch.int32, None)}


def _rows(kind, rng, M, K):
    if kind == "wide":
        # a twentieth of the values 2^-50 down (below the window: more levels), subnormals
        x = rng.standard_normal((M, K)).astype(np.float32)
        x[rng.random((M, K)) < 0.05] *= np.float32(2.0 ** -50)
        sub = rng.random((M, K)) < 0.01
        x[sub] = np.float32(2.0 ** -130) * rng.integers(1, 64, size=int(sub.sum())).astype(np.float32)
        return workloads.to_bf16_bits(x)
    return workloads.to_bf16_bits((2.0 * rng.standard_normal((M, K))).astype(np.float32))


def _oracle_chain(x, dlt, norm, bits, gran, packed_parts, gammas, epi, ydt):
    """x', then each part's (Y, acc) from the oracle's separate calls."""
    if norm == "rms":
        xp, h = oracle.rmsnorm(x, dlt)
    elif norm == "layer":
        xp, h = oracle.layernorm(x, dlt)
    else:
        xp, h = x, x
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq, s = oracle.quantize_acts(h, bits=bits, gran=g)
    outs = []
    for pk, gm in zip(packed_parts, gammas):
        y, acc = oracle.forward(xq, bits, s, g, pk, gm, epi=oracle.EPI_RELU2 if epi else oracle.EPI_NONE,
                                y_dtype=YDT[ydt][1] if ydt != "i32" else oracle.F32)
        outs.append(acc if ydt == "i32" else y)
    return xp, outs


CASES = [
    # M, K, N, parts, norm, residual, bits, gran, epilogue, y, rows
    # with a norm: the norm + quantization kernel, then the decode GEMV on its codes
    (16, 2560, 2560, 3, "rms", True, 8, "token", False, "bf16", "gauss"),   # the stack's QKV
    (16, 2560, 6912, 1, "rms", True, 8, "token", True, "bf16", "gauss"),    # the stack's up
    (1, 2560, 6912, 1, "rms", False, 8, "token", True, "f32", "gauss"),
    (5, 4096, 512, 2, "rms", True, 4, "token", False, "f32", "gauss"),
    (16, 64, 48, 1, "rms", True, 8, "token", False, "i32", "gauss"),
    (9, 1024, 100, 1, "rms", False, 4, "token", False, "i32", "gauss"),
    (16, 2560, 256, 1, "rms", True, 8, "token", False, "i32", "wide"),
    (3, 4096, 128, 1, "rms", False, 8, "token", False, "i32", "wide"),
    # without: one launch, the GEMV's row prologue quantizes
    (16, 2560, 2560, 1, None, False, 8, "token", False, "bf16", "gauss"),
    (12, 2048, 384, 2, None, False, 4, "token", True, "f32", "gauss"),
    (16, 6912, 2560, 1, None, False, 8, "token", False, "bf16", "gauss"),
    # the layer norm, per-tensor scales, K > 4096 (the codes GEMV), M > 16 (the GEMM)
    (16, 2560, 2560, 3, "layer", True, 8, "token", False, "bf16", "gauss"),
    (16, 2560, 512, 1, "rms", True, 8, "tensor", False, "f32", "gauss"),
    (16, 6912, 2560, 1, "rms", True, 8, "token", False, "bf16", "gauss"),
    (40, 2560, 512, 2, "rms", True, 8, "token", False, "f32", "gauss"),
    (7, 2560, 256, 1, None, False, 8, "tensor", False, "i32", "gauss"),
]


@pytest.mark.parametrize("M,K,N,parts,norm,res,bits,gran,epi,ydt,kind", CASES)
def test_norm_forward_parity(M, K, N, parts, norm, res, bits, gran, epi, ydt, kind):
    rng = np.random.default_rng([61, M, K, N, parts, bits, int(res), len(str(norm))])
    x = _rows(kind, rng, M, K)
    dlt = _rows(kind, rng, M, K) if res else None
    W = [workloads.ternary_weights(rng, N, K) for _ in range(parts)]
    say("norm_forward", M, K, N, parts, norm, res, bits, gran, epi, ydt, kind)
    pk_dev, gm_dev = [], []
    for w in W:
        p, g_ = bl.quantize_weights(to_dev(w))
        pk_dev.append(p)
        gm_dev.append(g_)
    packed = torch.stack(pk_dev) if parts > 1 else pk_dev[0]
    gamma = torch.cat(gm_dev)
    xd = to_dev(x)
    xo = torch.empty_like(xd) if res else None
    y = bl.norm_forward(xd, packed, gamma, delta=to_dev(dlt) if res else None, x_out=xo,
                        norm=norm, bits=bits, gran=gran, epilogue="relu2" if epi else None,
                        out_dtype=YDT[ydt][0])
    torch.cuda.synchronize()
    refs = [oracle.quantize_weights(w) for w in W]
    xp, outs = _oracle_chain(x, dlt, norm, bits, gran, [r[0] for r in refs], [r[1] for r in refs],
                             epi, ydt)
    assert_same_bytes(to_host(xd), x, "X is read only")
    if res:
        assert_same_bytes(to_host(xo), xp, "x'")
    got = to_host(y).reshape(parts, M, N)
    for p in range(parts):
        if ydt == "f32":
            assert_y_matches(got[p], outs[p], "f32", "part %d" % p)
        else:
            assert_same_bytes(got[p], outs[p], "part %d" % p)


@pytest.mark.parametrize("M,K,N,bits,epi", [(5, 2560, 6912, 8, True), (16, 2560, 2560, 8, False),
                                            (16, 4096, 1000, 4, False), (8, 64, 16, 8, True),
                                            (13, 1024, 4096, 4, True), (16, 6912, 2560, 8, False),
                                            (7, 8192, 272, 4, True), (16, 4160, 48, 8, False)])
def test_forward_fused_row_prologue(M, K, N, bits, epi):
    """5..16 bf16 tokens, per-token scales: bitlinear_forward_fused quantizes in the GEMV's
    prologue, a wave per token row, up to K = 4096 (wider rows, also checked here, take
    the quantizer's own launch); the codes must be the activation quantizer's."""
    rng = np.random.default_rng([62, M, K, N, bits])
    x = workloads.to_bf16_bits((3.0 * rng.standard_normal((M, K))).astype(np.float32))
    W = workloads.ternary_weights(rng, N, K)
    say("forward_fused rows", M, K, N, bits, epi)
    packed, gamma = bl.quantize_weights(to_dev(W))
    y = bl.forward_fused(to_dev(x), packed, gamma, bits=bits, epilogue="relu2" if epi else None,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    p_ref, g_ref, _ = oracle.quantize_weights(W)
    xq, s = oracle.quantize_acts(x, bits=bits)
    y_ref, _ = oracle.forward(xq, bits, s, oracle.PER_TOKEN, p_ref, g_ref,
                              epi=oracle.EPI_RELU2 if epi else oracle.EPI_NONE)
    assert_y_matches(to_host(y), y_ref, "f32", "y")


def test_norm_forward_repeatable():
    # the same call twice: bit-identical outputs (exact sums, no atomics in the path)
    rng = np.random.default_rng(63)
    x = to_dev(_rows("gauss", rng, 16, 2560))
    d = to_dev(_rows("gauss", rng, 16, 2560))
    packed, gamma = bl.quantize_weights(to_dev(workloads.ternary_weights(rng, 2560, 2560)))
    outs = []
    for _ in range(2):
        xo = torch.empty_like(x)
        outs.append((bl.norm_forward(x, packed, gamma, delta=d, x_out=xo,
                                     out_dtype=torch.bfloat16), xo))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
