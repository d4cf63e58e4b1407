"""GPU parity of the glue between BitLinear layers (residual add + RMS norm) and of
the 30-layer 2B-shaped decode stack, layer by layer: every library call of a layer is
checked against the oracle fed the GPU's own inputs for that call."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _check_norm(x_in, delta, x_gpu, h_gpu, what):
    x_ref, h_ref = oracle.rmsnorm(x_in, delta)
    assert_same_bytes(x_gpu, x_ref, what + " residual")
    d = np.abs(h_gpu.astype(np.int32) - h_ref.astype(np.int32))
    # the fp64 sum of squares is reduced in another order than the oracle's: at most
    # one bf16 ulp, and (in practice) almost never
    assert d.max(initial=0) <= 1, what + ": h more than one bf16 ulp off"
    assert np.count_nonzero(d) <= max(1, h_ref.size // 100000), what + ": too many ulp flips"


@pytest.mark.parametrize("M,K,with_delta", [(16, 2560, True), (16, 6912, False), (3, 6912, True),
                                            (1, 8, False), (5, 4104, True), (2, 65536, True)])
def test_rmsnorm_parity(M, K, with_delta):
    rng = np.random.default_rng([M, K])
    x = workloads.to_bf16_bits((3.0 * rng.standard_normal((M, K))).astype(np.float32))
    dlt = (workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
           if with_delta else None)
    say("rmsnorm", M, K, with_delta)
    xd = to_dev(x)
    h = bl.rmsnorm(xd, to_dev(dlt) if with_delta else None)
    torch.cuda.synchronize()
    _check_norm(x, dlt, to_host(xd), to_host(h), "rmsnorm %dx%d" % (M, K))


def test_rmsnorm_zero_rows():
    x = np.zeros((4, 64), np.uint16)
    xd = to_dev(x)
    h = bl.rmsnorm(xd)
    torch.cuda.synchronize()
    assert not to_host(h).any()


@pytest.mark.parametrize("M,K,bits,gran,with_delta", [
    (16, 2560, 8, "token", True), (16, 6912, 8, "token", False), (3, 256, 4, "token", True),
    (5, 4096, 8, "tensor", True), (2, 65536, 8, "token", False), (1, 16, 4, "tensor", False)])
def test_rmsnorm_quantize_parity(M, K, bits, gran, with_delta):
    rng = np.random.default_rng([M, K, bits])
    x = workloads.to_bf16_bits((2.0 * rng.standard_normal((M, K))).astype(np.float32))
    dlt = (workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
           if with_delta else None)
    say("rmsnorm_quantize", M, K, bits, gran, with_delta)
    xd = to_dev(x)
    h, xq, sc = bl.rmsnorm_quantize(xd, to_dev(dlt) if with_delta else None, bits=bits, gran=gran)
    torch.cuda.synchronize()
    hh = to_host(h)
    _check_norm(x, dlt, to_host(xd), hh, "rmsnorm_quantize %dx%d" % (M, K))
    # the codes and scales are the quantizer's, applied to the GPU's own h
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts(hh, bits=bits, gran=g)
    assert_same_bytes(to_host(xq), xq_ref, "codes")
    assert_same_bytes(to_host(sc).view(np.uint32), s_ref.view(np.uint32), "scales")


def _layer_weights(layer):
    codes = workloads.stack_layer_codes(3, layer)
    out = {}
    for name, c in codes.items():
        W = c.astype(np.float32)
        packed, gamma = bl.quantize_weights(to_dev(W))
        p_ref, g_ref, _ = oracle.quantize_weights(W)
        out[name] = (packed, gamma, p_ref, g_ref)
    torch.cuda.synchronize()
    for name, (packed, gamma, p_ref, g_ref) in out.items():
        assert_same_bytes(to_host(packed), p_ref, "layer %d %s packed" % (layer, name))
    return out


def _plain(hq, hs, h_host, packed, gamma, p_ref, g_ref, epi, what):
    """A BitLinear on the fused norm's codes; the oracle quantizes the same h itself."""
    y = bl.forward(hq, hs, packed, gamma, epilogue=epi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y_ref, _, _, _ = oracle.bitlinear(h_host, p_ref, g_ref,
                                      epi=oracle.EPI_RELU2 if epi else oracle.EPI_NONE,
                                      y_dtype=oracle.BF16)
    assert_same_bytes(to_host(y), y_ref, what)
    return y


def _fused(h_dev, packed, gamma, p_ref, g_ref, epi, what):
    """One BitLinear on the GPU, checked against the oracle on the same bf16 input."""
    y = bl.forward_fused(h_dev, packed, gamma, epilogue=epi, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    h = to_host(h_dev)
    y_ref, _, _, _ = oracle.bitlinear(h, p_ref, g_ref, epi=oracle.EPI_RELU2 if epi else oracle.EPI_NONE,
                                      y_dtype=oracle.BF16)
    assert_same_bytes(to_host(y), y_ref, what)
    return y


def test_stack_first_layers_parity():
    """The 2B stack at batch 16, layers 0 and 1, in the calls the benchmark makes: RMS
    norm fused with the quantization of h, Q, K and V on those codes in one call (V feeds
    O), O, residual + RMS norm + quantization, up + ReLU^2 on the codes, down, residual."""
    H = workloads.HIDDEN
    x = workloads.stack_input(seed=3, m=16)
    xd = to_dev(x)
    delta = None
    for layer in range(2):
        say("stack layer", layer)
        w = _layer_weights(layer)
        x_in = to_host(xd)
        d_in = to_host(delta) if delta is not None else None
        h, hq, hs = bl.rmsnorm_quantize(xd, delta)
        torch.cuda.synchronize()
        hh = to_host(h)
        _check_norm(x_in, d_in, to_host(xd), hh, "layer %d norm 1" % layer)
        pq, gq, pq_ref, gq_ref = w["qkv"]
        # Q, K and V in one call: three 2560-row parts of the one QKV tensor (one gamma)
        qkv = bl.forward_multi(hq, hs, pq.view(3, H, pq.shape[1]), gq.expand(3).contiguous(),
                               out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for part, name in enumerate("QKV"):
            y_ref, _, _, _ = oracle.bitlinear(hh, pq_ref[part * H:(part + 1) * H], gq_ref,
                                              epi=oracle.EPI_NONE, y_dtype=oracle.BF16)
            assert_same_bytes(to_host(qkv[part]), y_ref, "layer %d %s" % (layer, name))
        v = qkv[2]
        po, go, po_ref, go_ref = w["o"]
        o = _fused(v, po, go, po_ref, go_ref, None, "layer %d O" % layer)
        x_in = to_host(xd)
        h2, h2q, h2s = bl.rmsnorm_quantize(xd, o)
        torch.cuda.synchronize()
        h2h = to_host(h2)
        _check_norm(x_in, to_host(o), to_host(xd), h2h, "layer %d norm 2" % layer)
        pu, gu, pu_ref, gu_ref = w["up"]
        u = _plain(h2q, h2s, h2h, pu, gu, pu_ref, gu_ref, "relu2", "layer %d up" % layer)
        pd, gd, pd_ref, gd_ref = w["down"]
        delta = _fused(u, pd, gd, pd_ref, gd_ref, None, "layer %d down" % layer)
        assert np.isfinite(workloads.bf16_bits_to_f32(to_host(delta))).all()
