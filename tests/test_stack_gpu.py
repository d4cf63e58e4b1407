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
from gpu_util import assert_same_bytes, bits32, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _check_norm(x_in, delta, x_gpu, h_gpu, what):
    """The residual and h bit-exact against the oracle (S, the sum of squares, is exact on
    both sides, so no reduction order can move a bit).  Returns the oracle's (x', h)."""
    x_ref, h_ref = oracle.rmsnorm(x_in, delta)
    assert_same_bytes(x_gpu, x_ref, what + " residual")
    assert_same_bytes(h_gpu, h_ref, what + " h")
    return x_ref, h_ref


def _wide_rows(rng, M, K):
    """Gaussian bf16 rows with a twentieth of the values scaled down by 2^-50 (their squares
    lie more than 2^80 below the largest: the exact sum's slow path), a few subnormals and
    zeros."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    far = rng.random((M, K)) < 0.05
    x[far] *= np.float32(2.0 ** -50)
    sub = rng.random((M, K)) < 0.01
    x[sub] = np.float32(2.0 ** -130) * rng.integers(1, 64, size=int(sub.sum())).astype(np.float32)
    x[rng.random((M, K)) < 0.01] = 0.0
    return workloads.to_bf16_bits(x)


@pytest.mark.parametrize("M,K,with_delta,wide", [
    (16, 2560, True, False), (16, 6912, False, False), (3, 6912, True, False), (1, 8, False, False),
    (5, 4104, True, False), (2, 65536, True, False), (7, 2560, False, True), (3, 4104, True, True),
    (2, 65536, False, True)])
def test_rmsnorm_parity(M, K, with_delta, wide):
    rng = np.random.default_rng([M, K, int(wide)])
    x = (_wide_rows(rng, M, K) if wide else
         workloads.to_bf16_bits((3.0 * rng.standard_normal((M, K))).astype(np.float32)))
    dlt = (workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
           if with_delta else None)
    if wide and with_delta:
        dlt = _wide_rows(rng, M, K)
    say("rmsnorm", M, K, with_delta, wide)
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


@pytest.mark.parametrize("M,K,bits,gran,with_delta,wide", [
    (16, 2560, 8, "token", True, False), (16, 6912, 8, "token", False, False),
    (3, 256, 4, "token", True, False), (5, 4096, 8, "tensor", True, False),
    (2, 65536, 8, "token", False, False), (1, 16, 4, "tensor", False, False),
    (6, 2560, 8, "token", False, True), (4, 6912, 4, "token", True, True),
    (3, 2560, 8, "tensor", False, True)])
def test_rmsnorm_quantize_parity(M, K, bits, gran, with_delta, wide):
    rng = np.random.default_rng([M, K, bits, int(wide)])
    x = (_wide_rows(rng, M, K) if wide else
         workloads.to_bf16_bits((2.0 * rng.standard_normal((M, K))).astype(np.float32)))
    dlt = (workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
           if with_delta else None)
    say("rmsnorm_quantize", M, K, bits, gran, with_delta, wide)
    xd = to_dev(x)
    h, xq, sc = bl.rmsnorm_quantize(xd, to_dev(dlt) if with_delta else None, bits=bits, gran=gran)
    torch.cuda.synchronize()
    _, h_ref = _check_norm(x, dlt, to_host(xd), to_host(h), "rmsnorm_quantize %dx%d" % (M, K))
    g = oracle.PER_TOKEN if gran == "token" else oracle.PER_TENSOR
    xq_ref, s_ref = oracle.quantize_acts(h_ref, bits=bits, gran=g)
    assert_same_bytes(to_host(xq), xq_ref, "codes")
    assert_same_bytes(bits32(to_host(sc)), bits32(s_ref), "scales")


def _oracle_layer(x, delta, w):
    """One block of the stack in the oracle, from its own previous results."""
    H = workloads.HIDDEN
    bf = dict(y_dtype=oracle.BF16)
    r = {}
    r["x1"], r["h1"] = oracle.rmsnorm(x, delta)
    r["h1q"], r["h1s"] = oracle.quantize_acts(r["h1"], bits=8)
    _, pq, gq = w["qkv"]
    for part, name in enumerate("QKV"):
        r[name], _ = oracle.forward(r["h1q"], 8, r["h1s"], oracle.PER_TOKEN,
                                    pq[part * H:(part + 1) * H], gq, **bf)
    _, po, go = w["o"]
    r["O"], _, _, _ = oracle.bitlinear(r["V"], po, go, **bf)
    r["x2"], r["h2"] = oracle.rmsnorm(r["x1"], r["O"])
    r["h2q"], r["h2s"] = oracle.quantize_acts(r["h2"], bits=8)
    _, pu, gu = w["up"]
    r["up"], _ = oracle.forward(r["h2q"], 8, r["h2s"], oracle.PER_TOKEN, pu, gu,
                                epi=oracle.EPI_RELU2, **bf)
    _, pd, gd = w["down"]
    r["down"], _, _, _ = oracle.bitlinear(r["up"], pd, gd, **bf)
    return r


def _layer_weights(layer):
    """One block's packed weights on the GPU and in the oracle (checked equal)."""
    codes = workloads.stack_layer_codes(3, layer)
    w = {}
    for name, c in codes.items():
        W = c.astype(np.float32)
        packed, gamma = bl.quantize_weights(to_dev(W))
        p_ref, g_ref, _ = oracle.quantize_weights(W)
        w[name] = ((packed, gamma), p_ref, g_ref)
    torch.cuda.synchronize()
    for name, ((packed, gamma), p_ref, g_ref) in w.items():
        assert_same_bytes(to_host(packed), p_ref, "layer %d %s packed" % (layer, name))
        assert_same_bytes(bits32(to_host(gamma)), bits32(np.float32(g_ref).reshape(1)),
                          "layer %d %s gamma" % (layer, name))
    return w


@pytest.mark.timeout(1200)
def test_stack_30_layers_parity():
    """The 2B stack at batch 16, all 30 layers, in the calls the benchmark makes: RMS norm
    fused with the quantization of h, Q, K and V on those codes in one call (V feeds O),
    O, residual + RMS norm + quantization, up + ReLU^2 on the codes, down, residual
    ("BitNet 2B4T Guide", "End-to-End PyTorch Implementation": the block's norm -> QKV
    -> O -> norm -> FFN chain).  The oracle runs its own chain from the same x0 and
    weights; every GPU result of every layer (residual stream, h, codes, scales, each
    projection's output) is compared with the oracle's, bit for bit: zero code flips end
    to end."""
    H = workloads.HIDDEN
    x = workloads.stack_input(seed=3, m=16)
    xd = to_dev(x)
    x_ref = x.copy()
    delta, d_ref = None, None
    compared = 0
    for layer in range(workloads.LAYERS_2B):
        say("stack layer", layer)
        w = _layer_weights(layer)
        ref = _oracle_layer(x_ref, d_ref, w)
        (pq, gq), _, _ = w["qkv"]
        h, hq, hs = bl.rmsnorm_quantize(xd, delta)
        qkv = bl.forward_multi(hq, hs, pq.view(3, H, pq.shape[1]), gq.expand(3).contiguous(),
                               out_dtype=torch.bfloat16)
        x1 = to_host(xd)
        (po, go), _, _ = w["o"]
        o = bl.forward_fused(qkv[2], po, go, out_dtype=torch.bfloat16)
        h2, h2q, h2s = bl.rmsnorm_quantize(xd, o)
        (pu, gu), _, _ = w["up"]
        u = bl.forward(h2q, h2s, pu, gu, epilogue="relu2", out_dtype=torch.bfloat16)
        (pd, gd), _, _ = w["down"]
        delta = bl.forward_fused(u, pd, gd, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        got = {"x1": x1, "h1": to_host(h), "h1q": to_host(hq), "h1s": bits32(to_host(hs)),
               "Q": to_host(qkv[0]), "K": to_host(qkv[1]), "V": to_host(qkv[2]),
               "O": to_host(o), "x2": to_host(xd), "h2": to_host(h2), "h2q": to_host(h2q),
               "h2s": bits32(to_host(h2s)), "up": to_host(u), "down": to_host(delta)}
        ref["h1s"] = bits32(ref["h1s"])
        ref["h2s"] = bits32(ref["h2s"])
        for key, val in got.items():
            assert_same_bytes(val, ref[key], "layer %d %s" % (layer, key))
            compared += val.size
        x_ref, d_ref = ref["x2"], ref["down"]
    # the stream after the last block's residual add
    xf, _ = oracle.rmsnorm(x_ref, d_ref)
    xf_gpu = xd.clone()
    bl.rmsnorm(xf_gpu, delta)
    torch.cuda.synchronize()
    assert_same_bytes(to_host(xf_gpu), xf, "final residual stream")
    assert np.isfinite(workloads.bf16_bits_to_f32(xf)).all()
    say("stack: %d values compared over %d layers, 0 differ" % (compared, workloads.LAYERS_2B))


@pytest.mark.timeout(1200)
def test_stack_30_layers_fused_parity():
    """The same 30-layer stack in the benchmark's fused calls: residual add + RMS norm +
    quantization + Q, K, V in one call (bitlinear_norm_forward, three parts), O quantizing
    its own input, residual add + RMS norm + quantization + up (+ReLU^2) in one call,
    down quantizing its own input; the residual stream alternates between two buffers.
    Every value these calls write -- the stream after each add, Q, K, V, O, up, down --
    is compared with the oracle's chain from the same x0 and weights, bit for bit, and
    the final stream after the last residual add."""
    H = workloads.HIDDEN
    x = workloads.stack_input(seed=3, m=16)
    x0 = to_dev(x)
    bufs = (torch.empty_like(x0), torch.empty_like(x0))
    cur, delta = x0, None
    x_ref, d_ref = x.copy(), None
    compared = 0
    for layer in range(workloads.LAYERS_2B):
        say("fused stack layer", layer)
        w = _layer_weights(layer)
        ref = _oracle_layer(x_ref, d_ref, w)
        (pq, gq), _, _ = w["qkv"]
        nxt = bufs[0] if cur is not bufs[0] else bufs[1]
        qkv = bl.norm_forward(cur, pq.view(3, H, pq.shape[1]), gq.expand(3).contiguous(),
                              delta=delta, x_out=nxt if delta is not None else None,
                              out_dtype=torch.bfloat16)
        cur = nxt if delta is not None else cur
        x1 = to_host(cur)
        (po, go), _, _ = w["o"]
        o = bl.forward_fused(qkv[2], po, go, out_dtype=torch.bfloat16)
        (pu, gu), _, _ = w["up"]
        nxt = bufs[0] if cur is not bufs[0] else bufs[1]
        u = bl.norm_forward(cur, pu, gu, delta=o, x_out=nxt, epilogue="relu2",
                            out_dtype=torch.bfloat16)
        cur = nxt
        (pd, gd), _, _ = w["down"]
        delta = bl.forward_fused(u, pd, gd, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        got = {"x1": x1, "Q": to_host(qkv[0]), "K": to_host(qkv[1]), "V": to_host(qkv[2]),
               "O": to_host(o), "x2": to_host(cur), "up": to_host(u), "down": to_host(delta)}
        for key, val in got.items():
            assert_same_bytes(val, ref[key], "layer %d %s" % (layer, key))
            compared += val.size
        x_ref, d_ref = ref["x2"], ref["down"]
    xf, _ = oracle.rmsnorm(x_ref, d_ref)
    bl.rmsnorm(cur, delta)
    torch.cuda.synchronize()
    assert_same_bytes(to_host(cur), xf, "final residual stream")
    say("fused stack: %d values compared over %d layers, 0 differ" % (compared, workloads.LAYERS_2B))
