"""GPU parity of the glue between BitLinear layers (residual add + RMS norm) and of
the 2B-shaped decode stack: the oracle runs the same calls on its own, from the same
seeded inputs and weights, and every GPU result is compared with the oracle's."""
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
    """The residual bit-exact; h within one bf16 ulp of the oracle's (the fp64 sum of
    squares is reduced in another order: rarely a last-bit difference in r).  Returns
    the oracle's (x', h) and whether h is bit-identical."""
    x_ref, h_ref = oracle.rmsnorm(x_in, delta)
    assert_same_bytes(x_gpu, x_ref, what + " residual")
    d = np.abs(h_gpu.astype(np.int32) - h_ref.astype(np.int32))
    assert d.max(initial=0) <= 1, what + ": h more than one bf16 ulp off"
    assert np.count_nonzero(d) <= max(1, h_ref.size // 100000), what + ": too many ulp flips"
    return x_ref, h_ref, not d.any()


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
    _, h_ref, same = _check_norm(x, dlt, to_host(xd), hh, "rmsnorm_quantize %dx%d" % (M, K))
    # the codes and scales are the quantizer's of the oracle's h: exact on every row whose
    # h is bit-identical (per tensor: only if all of h is)
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts(h_ref, bits=bits, gran=g)
    rows = np.all(hh == h_ref, axis=1) if gran == "token" else np.full(M, same)
    if not rows.all():
        say("rmsnorm_quantize: h differs by one ulp in rows", np.nonzero(~rows)[0], "(not compared)")
    assert_same_bytes(to_host(xq)[rows], xq_ref[rows], "codes")
    sc_h = to_host(sc).view(np.uint32)
    s_ref_u = s_ref.view(np.uint32)
    assert_same_bytes(sc_h[rows] if gran == "token" else sc_h[:1] if same else sc_h[:0],
                      s_ref_u[rows] if gran == "token" else s_ref_u[:1] if same else s_ref_u[:0],
                      "scales")


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


def test_stack_first_layers_parity():
    """The 2B stack at batch 16, layers 0 and 1, in the calls the benchmark makes: RMS
    norm fused with the quantization of h, Q, K and V on those codes in one call (V feeds
    O), O, residual + RMS norm + quantization, up + ReLU^2 on the codes, down, residual.
    The oracle runs the same two layers on its own from the same x0 and weights; every
    GPU result is compared with the oracle's, bit for bit.  Should a norm's h ever differ
    by its documented ulp, the comparison stops there: everything after depends on h."""
    H = workloads.HIDDEN
    x = workloads.stack_input(seed=3, m=16)
    xd = to_dev(x)
    x_ref = x.copy()
    delta, d_ref = None, None
    bf = dict(y_dtype=oracle.BF16)
    for layer in range(2):
        say("stack layer", layer)
        w = _layer_weights(layer)
        h, hq, hs = bl.rmsnorm_quantize(xd, delta)
        torch.cuda.synchronize()
        x_ref, h_ref, same = _check_norm(x_ref, d_ref, to_host(xd), to_host(h), "layer %d norm 1" % layer)
        if not same:
            say("layer %d norm 1: h one ulp off the oracle's; chain comparison ends here" % layer)
            return
        pq, gq, pq_ref, gq_ref = w["qkv"]
        # Q, K and V in one call: three 2560-row parts of the one QKV tensor (one gamma)
        qkv = bl.forward_multi(hq, hs, pq.view(3, H, pq.shape[1]), gq.expand(3).contiguous(),
                               out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for part, name in enumerate("QKV"):
            y_ref, _, _, _ = oracle.bitlinear(h_ref, pq_ref[part * H:(part + 1) * H], gq_ref, **bf)
            assert_same_bytes(to_host(qkv[part]), y_ref, "layer %d %s" % (layer, name))
            if name == "V":
                v_ref = y_ref
        po, go, po_ref, go_ref = w["o"]
        o = bl.forward_fused(qkv[2], po, go, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        o_ref, _, _, _ = oracle.bitlinear(v_ref, po_ref, go_ref, **bf)
        assert_same_bytes(to_host(o), o_ref, "layer %d O" % layer)
        h2, h2q, h2s = bl.rmsnorm_quantize(xd, o)
        torch.cuda.synchronize()
        x_ref, h2_ref, same = _check_norm(x_ref, o_ref, to_host(xd), to_host(h2), "layer %d norm 2" % layer)
        if not same:
            say("layer %d norm 2: h one ulp off the oracle's; chain comparison ends here" % layer)
            return
        pu, gu, pu_ref, gu_ref = w["up"]
        u = bl.forward(h2q, h2s, pu, gu, epilogue="relu2", out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        u_ref, _, _, _ = oracle.bitlinear(h2_ref, pu_ref, gu_ref, epi=oracle.EPI_RELU2, **bf)
        assert_same_bytes(to_host(u), u_ref, "layer %d up" % layer)
        pd, gd, pd_ref, gd_ref = w["down"]
        delta = bl.forward_fused(u, pd, gd, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        d_ref, _, _, _ = oracle.bitlinear(u_ref, pd_ref, gd_ref, **bf)
        assert_same_bytes(to_host(delta), d_ref, "layer %d down" % layer)
        assert np.isfinite(workloads.bf16_bits_to_f32(d_ref)).all()
