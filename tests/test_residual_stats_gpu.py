"""GPU parity of the residual statistics path ("BitNet 2B4T Guide", "3. Sub-Layer
Normalization (SubLN)" and its block listing: a sub-layer's output is added to the
residual stream, and the next sub-layer RMS-normalizes the stream before its BitLinear
quantizes it).  bitlinear_forward_fused_residual adds a projection's output to the stream
and gathers the new rows' exact sum of squares and largest magnitude; the next
bitlinear_rmsnorm_forward_stats normalizes from those numbers instead of recomputing them.
The oracle runs the separate steps (fused forward, residual + RMS norm, quantization,
forward) from the same inputs; every output is compared bit for bit.  A producer's
`clear` zeroes another statistics buffer (in a stack, two alternate)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import ternary_weight_quantized_bitlinear_amd as bl
from gpu_util import assert_same_bytes, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _stream_rows(kind, rng, M, H):
    x = (2.0 * rng.standard_normal((M, H))).astype(np.float32)
    if kind == "wide":
        # a twentieth of the stream 2^-50 down: within a 16-column group, values far below
        # the group's largest go into the statistics on their own
        x[rng.random((M, H)) < 0.05] *= np.float32(2.0 ** -50)
    return workloads.to_bf16_bits(x)


@pytest.mark.parametrize("M,K1,H,parts,N2,bits,kind", [
    (16, 2560, 2560, 3, 2560, 8, "gauss"),   # O into the stream, then Q, K, V (the stack)
    (16, 6912, 2560, 1, 6912, 8, "gauss"),   # down into the stream, then up
    (1, 2560, 2560, 1, 6912, 8, "gauss"),    # one token: the M <= 4 prologue producer
    (5, 1024, 2048, 2, 512, 4, "wide"),      # int4 codes, far-below values in the stream
    (16, 2560, 4096, 1, 256, 8, "wide"),
    (16, 2560, 6912, 1, 2560, 8, "gauss"),   # consumer K = 6912: the norm kernel's path
    (24, 2560, 2560, 1, 512, 8, "gauss"),    # 24 tokens: both sides past the GEMV
    (7, 512, 1008, 1, 128, 8, "gauss"),      # width 63 x 16: the consumer past the GEMV (K % 64)
])
def test_residual_then_norm(M, K1, H, parts, N2, bits, kind):
    rng = np.random.default_rng([71, M, K1, H, parts, N2, bits])
    x = _stream_rows(kind, rng, M, H)
    V = workloads.to_bf16_bits(rng.standard_normal((M, K1)).astype(np.float32))
    W1 = (0.02 * rng.standard_normal((H, K1))).astype(np.float32)
    W2 = [workloads.ternary_weights(rng, N2, H) for _ in range(parts)]
    say("residual stats", M, K1, H, parts, N2, bits, kind)
    p1, g1 = bl.quantize_weights(to_dev(W1))
    p2l, g2l = zip(*[bl.quantize_weights(to_dev(w)) for w in W2])
    p2 = torch.stack(p2l) if parts > 1 else p2l[0]
    g2 = torch.cat(g2l)
    R = to_dev(x)
    stats = bl.new_norm_stats(M)
    y1 = torch.empty((M, H), dtype=torch.bfloat16, device=R.device)
    bl.forward_fused_residual(to_dev(V), p1, g1, R, stats=stats, y=y1, bits=bits)
    x1 = R.clone()
    Y2 = bl.rmsnorm_forward_stats(R, stats, p2, g2, bits=bits, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the oracle's separate steps
    q1, s1 = oracle.quantize_weights(W1)[:2]
    y1_ref, _, _, _ = oracle.bitlinear(V, q1, s1, bits=bits, y_dtype=oracle.BF16)
    x1_ref, h_ref = oracle.rmsnorm(x, y1_ref)
    xq, sc = oracle.quantize_acts(h_ref, bits=bits)
    assert_same_bytes(to_host(y1), y1_ref, "projection output")
    assert_same_bytes(to_host(x1), x1_ref, "residual stream")
    assert_same_bytes(to_host(R), x1_ref, "stream left as it was")
    got = to_host(Y2).reshape(parts, M, N2)
    for p, w in enumerate(W2):
        pk, gm, _ = oracle.quantize_weights(w)
        y2_ref, _ = oracle.forward(xq, bits, sc, oracle.PER_TOKEN, pk, gm, y_dtype=oracle.BF16)
        assert_same_bytes(got[p], y2_ref, "part %d" % p)
    # a later producer that fills another buffer clears this one
    other = bl.new_norm_stats(M)
    bl.forward_fused_residual(to_dev(V), p1, g1, R, stats=other, clear=stats, bits=bits)
    torch.cuda.synchronize()
    assert not to_host(stats).any(), "clear left statistics behind"
    assert to_host(other).any()


def test_residual_without_stats_and_repeated_cycles():
    # no statistics buffer: only the residual add; then three producer / reader cycles on
    # one buffer, each checked against a norm that computes its own sums
    rng = np.random.default_rng(72)
    M, H = 16, 2560
    x = _stream_rows("gauss", rng, M, H)
    W = (0.02 * rng.standard_normal((H, H))).astype(np.float32)
    p, g = bl.quantize_weights(to_dev(W))
    R = to_dev(x)
    V = to_dev(workloads.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32)))
    say("residual without stats")
    bl.forward_fused_residual(V, p, g, R)
    torch.cuda.synchronize()
    q, s = oracle.quantize_weights(W)[:2]
    y_ref, _, _, _ = oracle.bitlinear(to_host(V), q, s, y_dtype=oracle.BF16)
    x_ref, _ = oracle.rmsnorm(x, y_ref)
    assert_same_bytes(to_host(R), x_ref, "residual")
    stats = (bl.new_norm_stats(M), bl.new_norm_stats(M))
    for cycle in range(4):  # the two buffers alternate, each producer clearing the other
        say("cycle", cycle)
        fill, clear = stats[cycle % 2], stats[1 - cycle % 2]
        bl.forward_fused_residual(V, p, g, R, stats=fill, clear=clear)
        a = bl.rmsnorm_forward_stats(R, fill, p, g, out_dtype=torch.bfloat16)
        b = bl.norm_forward(R, p, g, norm="rms", out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), cycle
        assert not to_host(clear).any(), cycle
