"""Benchmark of the MI355X BitLinear forward pass.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs decode,chain,single,prefill,pack,cpu]

Headline (one JSON line on stdout): decode-GEMV HBM throughput on the BitNet 2B FFN
shapes at M=1 token, streamed.  One step = the FFN of 64 independent 2B-shaped layers
(64 distinct weight copies, 566 MB per step), each at decode time:
    x_b (bf16 [1, 2560])  --up 2560->6912, ReLU^2-->  h_b (bf16 [1, 6912])
                          --down 6912->2560-->         y_b (bf16 [1, 2560])
as two launches of bitlinear_forward_fused_batched (all 64 up projections, then all 64
down projections).  Each fuses per-token absmax int8 quantization of its input (for
down: the requantization of up's output), the ternary GEMV with int32 accumulation and
the rescale epilogue.  Consecutive steps cycle through 3 such sets (1.7 GB), so no
weights are still in the 256 MB Infinity Cache when they are read again and the stream
really comes from HBM.  Packed weights are pre-quantized (bitlinear_quantize_weights,
timed separately as the "pack" leg): the pages treat weights as static.

Inputs are resident in HBM before timing.  The K timed steps are captured in one HIP
graph and timed with HIP events on the stream the kernels run on.

value        = algorithmic bytes per step / time per step (GB/s, 1e9 B/s)
roofline     = the batched GEMV kernel against MI355X HBM (8 TB/s); traffic from the
               committed FETCH_SIZE/WRITE_SIZE counter summary while it matches the
               kernel sources
decode_chain = one layer's FFN step alone (two dependent 4.4 MB launches: latency-bound)
prefill      = the prefill GEMM leg: M=2048 tokens, int TOPS against int8 MFMA peak
backward     = the straight-through-estimator backward (dX, dW, dbias), TFLOP/s against
               the bf16 MFMA peak
parity_layer = the 8 x 256 -> 512 parity configuration, timed only
mfma_ceiling = MFMA-only loops on register operands with each GEMM's operand statistics
               (int8, FP4 x FP6, bf16): the matrix cores' rate on this chip, reported
               beside each GEMM's fraction of the published peak
hbm_read_ceiling = a read-only sweep of 16-byte loads over 1 GiB: the rate streaming
               reads reach on this chip, beside the decode kernel's fraction of 8 TB/s
cpu_baseline = the CPU oracle pinned to one core: one layer's decode FFN step (the
               headline's unit), plus the parity layer in full and samples of the
               prefill GEMM, the 30-layer stack and the 70B layer, extrapolated
stack_launches_us = (leg "launches", only when named) each call of the 2B stack's block
               at 16 tokens and at 1, repeated with rotated weights: per-launch costs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, TOPS (5.0 POP/s)
F6F4_PEAK_TOPS = 10100.0        # MI355X dense FP6/FP4 MFMA (10.1 PFLOP/s), the int4 path's units
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20          # Infinity Cache
METRIC = "BitLinear decode GEMV HBM GB/s + prefill GEMM int TOPS, % of MI355X roofline"
CSRC = os.path.join(ROOT, "ternary_weight_quantized_bitlinear_amd", "csrc")
# HBM traffic of the decode GEMV, from two rocprofv3 --pmc runs of the "traffic" leg
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_decode_2b_traffic.txt")
GEMV_SOURCES = ("gemv.hip", "common.hpp")


def gemv_bytes(K: int, N: int) -> int:
    """Algorithmic bytes of one decode GEMV: packed W + bf16 x + bf16 y + gamma."""
    return N * K // 4 + 2 * K + 2 * N + 4


def gemv_source_digest() -> str:
    """Digest of the sources the decode GEMV kernel is built from."""
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode GEMV launch from the committed counter summary, or None when
    there is none or the kernel sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_digest") != gemv_source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def graph_time_ms(torch, fn, replays: int, warm: int = 2, steady_ms: float = 0.0):
    """Capture fn() in a HIP graph; return (ms per replay, graph) over `replays` replays.

    steady_ms > 0: before timing, untimed replays keep the GPU busy for at least that
    long, so that clocks and memory have left their idle states whatever the replay's
    length.  The timed replays are queued behind a short spin kernel, so the first one is
    already submitted when the start event fires: the host's submission time is not
    timed."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up outside capture (allocations, lazy init)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if steady_ms > 0:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        g.replay()
        w1.record(stream)
        torch.cuda.synchronize()
        one = max(w0.elapsed_time(w1), 1e-3)
        for _ in range(int(steady_ms / one) + 1):
            g.replay()
        torch.cuda._sleep(2_000_000)  # ~1 ms of spinning while the timed replays queue up
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / replays, g


def make_weight_copies(torch, bl, W0, copies, seed):
    """Copy 0: the seeded host weights; the others: distinct uniform-ternary tensors drawn
    on the device; all packed by bitlinear_quantize_weights."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    N, K = W0.shape
    out = []
    for c in range(copies):
        if c == 0:
            W = torch.from_numpy(W0).to(dev)
        else:
            W = torch.randint(-1, 2, (N, K), device=dev, generator=gen, dtype=torch.int8).float()
        out.append(bl.quantize_weights(W))
        del W
    torch.cuda.synchronize()
    return out


def leg_decode(torch, bl, steps, warmup, copies):
    import workloads
    dev = torch.device("cuda:0")
    (K1, N1), (K2, N2) = workloads.SHAPE_UP, workloads.SHAPE_DOWN
    W_up, x = workloads.decode_gemv(seed=1, shape=workloads.SHAPE_UP)
    W_dn, _ = workloads.decode_gemv(seed=1, shape=workloads.SHAPE_DOWN)
    up = make_weight_copies(torch, bl, W_up, copies, 11)
    dn = make_weight_copies(torch, bl, W_dn, copies, 12)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    h = torch.empty((1, N1), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, N2), dtype=torch.bfloat16, device=dev)

    def step(i):
        pu, gu = up[i % copies]
        pd, gd = dn[i % copies]
        bl.forward_fused(xd, pu, gu, epilogue="relu2", out=h)
        bl.forward_fused(h, pd, gd, out=y)

    def run_k():
        for i in range(steps):
            step(i)

    # warm-up steps (untimed), then exactly `steps` steps in one graph
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms_total, _ = graph_time_ms(torch, run_k, replays=1, warm=1)
    ms_step = ms_total / steps
    step_bytes = gemv_bytes(K1, N1) + gemv_bytes(K2, N2)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    per_launch_us = ms_step * 1e3 / 2
    return {
        "ms_per_step": ms_step, "gbs": gbs, "step_bytes": step_bytes,
        "per_launch_us": per_launch_us, "launches_per_step": 2,
        "bytes_per_launch": step_bytes / 2, "weight_copies": copies,
        "rotation_bytes": copies * (N1 * K1 // 4 + N2 * K2 // 4),
        "x": x, "W_up": W_up, "W_dn": W_dn,
    }


def make_weight_batch(torch, bl, W0, batch, seed):
    """[batch, N, K/4] packed weights + gamma [batch]: problem 0 from the seeded host
    weights, the others distinct uniform-ternary tensors drawn on the device."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    N, K = W0.shape
    packed = torch.empty((batch, N, K // 4), dtype=torch.uint8, device=dev)
    gamma = torch.empty((batch,), dtype=torch.float32, device=dev)
    for b in range(batch):
        if b == 0:
            W = torch.from_numpy(W0).to(dev)
        else:
            W = torch.randint(-1, 2, (N, K), device=dev, generator=gen, dtype=torch.int8).float()
        bl.quantize_weights(W, out=(packed[b], gamma[b:b + 1]))
        del W
    torch.cuda.synchronize()
    return packed, gamma


def leg_decode_stream(torch, bl, steps, warmup, batch, sets=3):
    """Headline: the FFN decode step of `batch` independent 2B-shaped layers, M=1 each.
    Per step two launches of bitlinear_forward_fused_batched: up (x_b -> h_b, ReLU^2) over
    all layers, then down (h_b requantized -> y_b).  Consecutive steps cycle through
    `sets` independent weight sets (3 x 566 MB), so that no weights can still sit in the
    256 MB Infinity Cache when they are read again: every step streams its weights from
    HBM.  (With one set, the whole-line kernel's nontemporal up loads leave most of the
    down weights cached between steps, which would overstate the HBM rate.)  The K timed
    steps are one HIP graph."""
    import workloads
    dev = torch.device("cuda:0")
    (K1, N1), (K2, N2) = workloads.SHAPE_UP, workloads.SHAPE_DOWN
    W_up, x = workloads.decode_gemv(seed=1, shape=workloads.SHAPE_UP)
    W_dn, _ = workloads.decode_gemv(seed=1, shape=workloads.SHAPE_DOWN)
    wsets = [make_weight_batch(torch, bl, W_up, batch, 41 + 10 * i) +
             make_weight_batch(torch, bl, W_dn, batch, 42 + 10 * i) for i in range(sets)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(43)
    X = torch.randn((batch, 1, K1), device=dev, generator=gen).to(torch.bfloat16)
    X[0, 0] = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)[0]
    h = torch.empty((batch, 1, N1), dtype=torch.bfloat16, device=dev)
    y = torch.empty((batch, 1, N2), dtype=torch.bfloat16, device=dev)

    def step(i):
        pu, gu, pd, gd = wsets[i % sets]
        bl.forward_fused_batched(X, pu, gu, epilogue="relu2", out=h)
        bl.forward_fused_batched(h, pd, gd, out=y)

    def run_k():
        for i in range(steps):
            step(i)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # exactly `steps` steps timed, after at least 300 ms of untimed streaming
    ms_total, g = graph_time_ms(torch, run_k, replays=1, warm=1, steady_ms=300.0)
    ms_step = ms_total / steps
    # context only: the same graph replayed 5 more times, each timed on its own
    rep = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(2_000_000)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        rep.append(e0.elapsed_time(e1) / steps)
    step_bytes = batch * (gemv_bytes(K1, N1) + gemv_bytes(K2, N2))
    return {"ms_per_step": ms_step, "gbs": step_bytes / (ms_step * 1e-3) / 1e9,
            "step_bytes": step_bytes, "per_launch_us": ms_step * 1e3 / 2,
            "bytes_per_launch": step_bytes / 2, "batch": batch, "sets": sets, "x": x,
            "W_up": W_up, "W_dn": W_dn, "repeat_ms_per_step": rep}


def leg_decode_single(torch, bl, copies=64, reps=200):
    """Each GEMV alone (up, then down), rotating copies, graph-captured: per-launch time."""
    import workloads
    dev = torch.device("cuda:0")
    res = {}
    for name, shape, epi in (("up", workloads.SHAPE_UP, "relu2"),
                             ("down", workloads.SHAPE_DOWN, None)):
        K, N = shape
        W, x = workloads.decode_gemv(seed=1, shape=shape)
        ws = make_weight_copies(torch, bl, W, copies, 21)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)

        def run():
            for i in range(reps):
                p, g = ws[i % copies]
                bl.forward_fused(xd, p, g, epilogue=epi, out=y)

        ms, _ = graph_time_ms(torch, run, replays=1)
        us = ms * 1e3 / reps
        res[name] = {"us_per_launch": us, "gbs": gemv_bytes(K, N) / (us * 1e-6) / 1e9}
        del ws
    return res


def leg_prefill(torch, bl, reps=20):
    """Prefill: M=2048 tokens at the 2B FFN shapes, bf16 Y (ReLU^2 on up).  "gemm": the
    forward on int8 per-token activations (bitlinear_forward); "step": the whole layer on
    bf16 X (bitlinear_forward_fused: quantization straight into the GEMM's operand form).
    "int4": the same two calls with 4-bit activations, whose contraction runs exactly on
    the FP6 x FP4 matrix cores (their operand preparation is inside both timings)."""
    import workloads
    dev = torch.device("cuda:0")
    res = {}
    tot_ops, tot_gemm_ms, tot_step_ms = 0.0, 0.0, 0.0
    for name, shape, epi in (("up", workloads.SHAPE_UP, "relu2"),
                             ("down", workloads.SHAPE_DOWN, None)):
        K, N = shape
        W, X = workloads.prefill_gemm(seed=2, shape=shape)
        packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(dev))
        Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
        M = X.shape[0]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ops = 2.0 * M * N * K
        for bits in (8, 4):
            xq, s = bl.quantize_acts(Xd, bits=bits)
            # workspaces allocated once, as a serving loop would
            ws = torch.empty(bl.workspace_size(bl.BL_OP_FORWARD, M, N, K, bits), dtype=torch.uint8,
                             device=dev)
            wsf = torch.empty(bl.workspace_size(bl.BL_OP_FORWARD_FUSED, M, N, K, bits),
                              dtype=torch.uint8, device=dev)

            def gemm():
                for _ in range(reps):
                    bl.forward(xq, s, packed, gamma, bits=bits, epilogue=epi, out=y, workspace=ws)

            def stepf():
                for _ in range(reps):
                    bl.forward_fused(Xd, packed, gamma, bits=bits, epilogue=epi, out=y,
                                     workspace=wsf)

            ms_gemm, _ = graph_time_ms(torch, gemm, replays=1)
            ms_step, _ = graph_time_ms(torch, stepf, replays=1)
            ms_gemm /= reps
            ms_step /= reps
            r = {"gemm_us": ms_gemm * 1e3, "gemm_tops": ops / (ms_gemm * 1e-3) / 1e12,
                 "step_us": ms_step * 1e3, "step_tops": ops / (ms_step * 1e-3) / 1e12}
            if bits == 8:
                res[name] = {"M": M, "K": K, "N": N, **r}
                tot_ops += ops
                tot_gemm_ms += ms_gemm
                tot_step_ms += ms_step
            else:
                res.setdefault("int4", {})[name] = r
                t4 = res["int4"]
                t4["_ms"] = t4.get("_ms", 0.0) + ms_gemm
            del xq, ws, wsf
    tops = tot_ops / (tot_gemm_ms * 1e-3) / 1e12
    res["gemm_tops"] = tops
    res["gemm_frac"] = tops / INT8_PEAK_TOPS
    res["step_tops"] = tot_ops / (tot_step_ms * 1e-3) / 1e12
    t4 = res["int4"]
    t4["gemm_tops"] = tot_ops / (t4.pop("_ms") * 1e-3) / 1e12
    t4["mfma"] = "fp6 x fp4 scaled MFMA (exact): 32x32x64 on up, 16x16x128 in balanced tiles on down"
    t4["peak_tops"] = F6F4_PEAK_TOPS
    t4["frac"] = t4["gemm_tops"] / F6F4_PEAK_TOPS
    return res


def leg_traffic(torch, bl, reps=4, batch=64):
    """Eager launches for the counter runs (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE):
    the two streamed decode launches of the headline (batched fused GEMV over `batch`
    layers), and a plain int32 streaming kernel of known size (256 MiB read, 256 MiB
    written) that calibrates what the counters report."""
    import workloads
    dev = torch.device("cuda:0")
    for name, shape, epi in (("up", workloads.SHAPE_UP, "relu2"),
                             ("down", workloads.SHAPE_DOWN, None)):
        K, N = shape
        W, x = workloads.decode_gemv(seed=1, shape=shape)
        packed, gamma = make_weight_batch(torch, bl, W, batch, 31)
        X = torch.randn((batch, 1, K), device=dev).to(torch.bfloat16)
        y = torch.empty((batch, 1, N), dtype=torch.bfloat16, device=dev)
        for _ in range(reps):
            bl.forward_fused_batched(X, packed, gamma, epilogue=epi, out=y)
        torch.cuda.synchronize()
        print("traffic leg: %d launches of the batched %s GEMV (%d layers, K=%d, N=%d), "
              "%d B algorithmic each" % (reps, name, batch, K, N, batch * gemv_bytes(K, N)),
              flush=True)
        del packed
    n = 64 << 20
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print("traffic leg: 4 launches of bitwise_not over %d B int32 (reads %d B, writes %d B)"
          % (4 * n, 4 * n, 4 * n), flush=True)
    print("traffic leg: gemv source digest %s" % gemv_source_digest(), flush=True)


def leg_70b(torch, bl, reps=5, err_rows=16):
    """70B-class FFN layer, int8 vs int4 activations (the a4.8 comparison): M=4096 tokens,
    K=8192, N=28672, 41 outlier channels x30, bf16 Y.  Per path: the GEMM on quantized
    activations (bitlinear_forward) and the fused quantize + GEMM (bitlinear_forward_fused),
    and the quantization error: ||Y - Y_ref||_F / ||Y_ref||_F over `err_rows` sampled tokens,
    Y_ref = X (gamma c)^T in float64 on the host."""
    import workloads
    dev = torch.device("cuda:0")
    codes, X = workloads.layer_70b()
    M, K = X.shape
    N = codes.shape[0]
    Wd = torch.from_numpy(codes).to(dev).float()
    packed, gamma = bl.quantize_weights(Wd)
    del Wd
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    rows = np.random.default_rng(7).choice(M, err_rows, replace=False)
    xr = workloads.bf16_bits_to_f32(X[rows]).astype(np.float64)
    g = float(gamma.cpu()[0])
    y_ref = (xr @ codes.T.astype(np.float64)) * g
    ref_norm = np.linalg.norm(y_ref)
    ops = 2.0 * M * N * K
    out = {"M": M, "K": K, "N": N, "int_ops": ops}
    for bits in (8, 4):
        xq, sc = bl.quantize_acts(Xd, bits=bits)
        ws = torch.empty(bl.workspace_size(bl.BL_OP_FORWARD, M, N, K, bits), dtype=torch.uint8,
                         device=dev)
        wsf = torch.empty(bl.workspace_size(bl.BL_OP_FORWARD_FUSED, M, N, K, bits), dtype=torch.uint8,
                          device=dev)

        def gemm():
            for _ in range(reps):
                bl.forward(xq, sc, packed, gamma, bits=bits, out=y, workspace=ws)

        def fused():
            for _ in range(reps):
                bl.forward_fused(Xd, packed, gamma, bits=bits, out=y, workspace=wsf)

        ms_g, _ = graph_time_ms(torch, gemm, replays=1)
        ms_f, _ = graph_time_ms(torch, fused, replays=1)
        ms_g /= reps
        ms_f /= reps
        yr = torch.from_numpy(rows).to(dev)
        yh = y.index_select(0, yr).float().cpu().numpy().astype(np.float64)
        peak = INT8_PEAK_TOPS if bits == 8 else F6F4_PEAK_TOPS
        out["int%d" % bits] = {
            "mfma": ("int8 16x16x64 in 128 x 448 tiles" if bits == 8
                     else "fp6 x fp4 32x32x64 (exact)"),
            "peak_tops": peak, "frac": ops / (ms_g * 1e-3) / 1e12 / peak,
            "gemm_us": ms_g * 1e3, "gemm_tops": ops / (ms_g * 1e-3) / 1e12,
            "fused_us": ms_f * 1e3, "fused_tops": ops / (ms_f * 1e-3) / 1e12,
            "act_bytes": M * K if bits == 8 else M * K // 2,
            "rel_fro_err": float(np.linalg.norm(yh - y_ref) / ref_norm)}
        del xq, ws, wsf
    out["err_sample"] = "%d token rows x all %d outputs vs float64 X (gamma c)^T" % (err_rows, N)

    # Hadamard rotation before the 4-bit activations (the a4.8 page's outlier
    # suppression), folded into both operands: the same weights rotated and ternarized
    # again (offline), the activations rotated and quantized in one pass, then the same
    # FP6 x FP4 GEMM.  Its error is taken against that path's own exact product
    # (X H)(gamma' c')^T / b, so that it isolates the activation quantization, as above.
    Wd = torch.from_numpy(codes).to(dev).float()
    pr, gr = bl.quantize_weights_rotated(Wd)
    del Wd
    b = bl.hadamard_block(K)
    xq, sc = bl.quantize_acts_rotated(Xd, bits=4)
    ws = torch.empty(bl.workspace_size(bl.BL_OP_FORWARD, M, N, K, 4), dtype=torch.uint8,
                     device=dev)

    def rot_gemm():
        for _ in range(reps):
            bl.forward(xq, sc, pr, gr, bits=4, out=y, workspace=ws)

    def rot_step():
        for _ in range(reps):
            bl.quantize_acts_rotated(Xd, bits=4, out=(xq, sc))
            bl.forward(xq, sc, pr, gr, bits=4, out=y, workspace=ws)

    ms_g = graph_time_ms(torch, rot_gemm, replays=1)[0] / reps
    ms_s = graph_time_ms(torch, rot_step, replays=1)[0] / reps
    yh = y.index_select(0, torch.from_numpy(rows).to(dev)).float().cpu().numpy().astype(np.float64)
    ph = pr.cpu().numpy()
    c_rot = (((ph[:, :, None] >> np.array([0, 2, 4, 6], np.uint8)) & 3).reshape(N, K)
             .astype(np.int8) - 1)
    y_rref = (_fwht_rows(xr, b) @ c_rot.T.astype(np.float64)) * float(gr.cpu()[0])
    out["int4_rotated"] = {
        "mfma": "fp6 x fp4 32x32x64 (exact)", "hadamard_block": b,
        "peak_tops": F6F4_PEAK_TOPS, "frac": ops / (ms_g * 1e-3) / 1e12 / F6F4_PEAK_TOPS,
        "gemm_us": ms_g * 1e3, "gemm_tops": ops / (ms_g * 1e-3) / 1e12,
        "step_us": ms_s * 1e3, "step_tops": ops / (ms_s * 1e-3) / 1e12,
        "rel_fro_err": float(np.linalg.norm(yh - y_rref) / np.linalg.norm(y_rref)),
        "err_ref": "float64 (X H)(gamma' c')^T / b, c' and gamma' the rotated weights' codes"}
    del xq, ws, pr
    return out


def _fwht_rows(x, b):
    """Rows of x (float64) times the block-diagonal unnormalized Hadamard matrix, blocks of
    b along the last axis (a reference: the order of the additions does not matter here)."""
    M, K = x.shape
    y = x.reshape(M, K // b, b).copy()
    h = 1
    while h < b:
        v = y.reshape(M, K // b, b // (2 * h), 2, h)
        lo, hi = v[:, :, :, 0, :].copy(), v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = lo + hi
        v[:, :, :, 1, :] = lo - hi
        h *= 2
    return y.reshape(M, K)


def leg_stack(torch, bl, steps=10, layers=30, batch=16):
    """The 2B-shaped decode stack: 30 blocks of QKV 2560->7680, O 2560->2560, up
    2560->6912 (+ReLU^2), down 6912->2560, batch 16 tokens, seed-fixed weights.  Per
    block: residual add + RMS norm + quantization + Q, K, V in one call (V feeds O)
    -> O -> residual add + RMS norm + quantization + up in one call -> down; O and down
    quantize their bf16 inputs themselves.  One step = all 30 blocks for the 16 tokens,
    the K steps in one graph.  The same block as separate calls (norm + quantization,
    then the projections) is timed beside it, and both must end on the same residual
    stream, bit for bit."""
    import workloads
    dev = torch.device("cuda:0")
    H = workloads.HIDDEN
    W = []
    wbytes = 0
    for layer in range(layers):
        codes = workloads.stack_layer_codes(3, layer)
        lw = {}
        for name, c in codes.items():
            Wd = torch.from_numpy(c).to(dev).float()
            lw[name] = bl.quantize_weights(Wd)
            wbytes += c.size // 4
            del Wd
        # the QKV tensor (one gamma) as three 2560-row parts of one input
        pq, gq = lw["qkv"]
        lw["qkv3"] = (pq.view(3, H, pq.shape[1]), gq.expand(3).contiguous())
        W.append(lw)
    torch.cuda.synchronize()
    x0 = torch.from_numpy(workloads.stack_input(seed=3, m=batch).view(np.int16)).to(dev).view(
        torch.bfloat16)
    x = x0.clone()
    h = torch.empty_like(x)
    hq = torch.empty((batch, H), dtype=torch.int8, device=dev)
    hs = torch.empty((batch,), dtype=torch.float32, device=dev)
    qkv = torch.empty((3, batch, H), dtype=torch.bfloat16, device=dev)
    v = qkv[2]
    o = torch.empty((batch, H), dtype=torch.bfloat16, device=dev)
    u = torch.empty((batch, workloads.FFN), dtype=torch.bfloat16, device=dev)
    d = torch.empty((batch, H), dtype=torch.bfloat16, device=dev)

    bufs = (torch.empty_like(x0), torch.empty_like(x0))
    nf_ws = torch.empty(max(bl.workspace_size(bl.BL_OP_NORM_FORWARD, batch, n, H)
                            for n in (H, workloads.FFN)), dtype=torch.uint8, device=dev)
    ff_ws = torch.empty(max(bl.workspace_size(bl.BL_OP_FORWARD_FUSED, batch, n, k)
                            for n, k in ((H, H), (H, workloads.FFN))), dtype=torch.uint8, device=dev)
    final = {}

    def step():
        # each sub-layer's input side in one call: residual add (into the other stream
        # buffer), RMS norm, quantization and the projections (Q, K, V in one call)
        cur, delta = x0, None
        for lw in W:
            pq3, gq3 = lw["qkv3"]
            nxt = bufs[0] if cur is not bufs[0] else bufs[1]
            bl.norm_forward(cur, pq3, gq3, delta=delta, x_out=nxt if delta is not None else None,
                            out=qkv, workspace=nf_ws)
            cur = nxt if delta is not None else cur
            bl.forward_fused(v, *lw["o"], out=o, workspace=ff_ws)
            nxt = bufs[0] if cur is not bufs[0] else bufs[1]
            bl.norm_forward(cur, *lw["up"], delta=o, x_out=nxt, epilogue="relu2", out=u,
                            workspace=nf_ws)
            cur = nxt
            bl.forward_fused(u, *lw["down"], out=d, workspace=ff_ws)
            delta = d
        bl.rmsnorm(cur, delta, out=h)  # the last residual
        final["x"] = cur

    def step_unfused():
        # the same block as separate calls: norm + quantization, then the projections
        x.copy_(x0)
        delta = None
        for lw in W:
            pq3, gq3 = lw["qkv3"]
            bl.rmsnorm_quantize(x, delta, out=(h, hq, hs))
            bl.forward_multi(hq, hs, pq3, gq3, out=qkv)  # Q, K, V: one call, V = qkv[2]
            bl.forward_fused(v, *lw["o"], out=o)
            bl.rmsnorm_quantize(x, o, out=(h, hq, hs))
            bl.forward(hq, hs, *lw["up"], epilogue="relu2", out=u)
            bl.forward_fused(u, *lw["down"], out=d)
            delta = d
        bl.rmsnorm(x, delta, out=h)  # the last residual

    def run():
        for _ in range(steps):
            step()

    def run_unfused():
        for _ in range(steps):
            step_unfused()

    step()
    step_unfused()
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(final["x"].float()).all())
    same = bool(torch.equal(final["x"].view(torch.int16), x.view(torch.int16)))
    ms, _ = graph_time_ms(torch, run, replays=1)
    ms /= steps
    ms_u, _ = graph_time_ms(torch, run_unfused, replays=1)
    ms_u /= steps
    return {"layers": layers, "batch": batch, "ms_per_step": ms, "tokens_per_s": batch / (ms * 1e-3),
            "weight_bytes_per_step": wbytes, "weight_gbs": wbytes / (ms * 1e-3) / 1e9,
            "library_calls_per_step": layers * 4 + 1, "output_finite": finite,
            "unfused_ms_per_step": ms_u, "unfused_library_calls_per_step": layers * 6 + 1,
            "fused_equals_unfused": same}


def leg_stack_launches(torch, bl, copies=24, reps=48):
    """Per-launch cost of each call of the 2B stack's block at batch 16 and at one token,
    each call repeated with `copies` weight sets rotated, graph-timed after 100 ms of
    untimed replays: the latency floor each of the stack's launches sits on.  Not in the
    default legs (name it in --legs)."""
    import workloads
    dev = torch.device("cuda:0")
    H, F = workloads.HIDDEN, workloads.FFN
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def wset(n, k):
        out = []
        for _ in range(copies):
            W = torch.randint(-1, 2, (n, k), device=dev, generator=gen).float()
            out.append(bl.quantize_weights(W))
            del W
        return out

    w_hh, w_fh, w_hf = wset(H, H), wset(F, H), wset(H, F)
    w_q3 = [(p.repeat(3, 1).view(3, H, p.shape[1]), g.expand(3).contiguous()) for p, g in w_hh]
    ws = torch.empty(max(bl.workspace_size(bl.BL_OP_FORWARD_FUSED, 16, H, F),
                         bl.workspace_size(bl.BL_OP_FORWARD, 16, F, H)) + 256,
                     dtype=torch.uint8, device=dev)
    res = {"copies": copies, "calls_per_graph": reps}
    for M in (16, 1):
        x = torch.randn((M, H), device=dev, generator=gen).to(torch.bfloat16)
        dl = torch.randn((M, H), device=dev, generator=gen).to(torch.bfloat16)
        u = torch.randn((M, F), device=dev, generator=gen).to(torch.bfloat16)
        xq, xs = bl.quantize_acts(x)
        uq, us = bl.quantize_acts(u)
        yH = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        yF = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        y3 = torch.empty((3, M, H), dtype=torch.bfloat16, device=dev)
        h = torch.empty_like(x)
        hq = torch.empty((M, H), dtype=torch.int8, device=dev)
        hs = torch.empty((M,), dtype=torch.float32, device=dev)
        cases = (
            ("rmsnorm_quantize 2560", lambda i: bl.rmsnorm_quantize(x, dl, out=(h, hq, hs))),
            ("qkv codes 2560->3x2560", lambda i: bl.forward_multi(xq, xs, *w_q3[i % copies], out=y3)),
            ("o bf16 2560->2560", lambda i: bl.forward_fused(x, *w_hh[i % copies], out=yH, workspace=ws)),
            ("up codes 2560->6912 relu2", lambda i: bl.forward(xq, xs, *w_fh[i % copies], epilogue="relu2",
                                                              out=yF, workspace=ws)),
            ("quantize_acts 6912", lambda i: bl.quantize_acts(u, out=(uq, us))),
            ("down codes 6912->2560", lambda i: bl.forward(uq, us, *w_hf[i % copies], out=yH, workspace=ws)),
            ("down bf16 6912->2560", lambda i: bl.forward_fused(u, *w_hf[i % copies], out=yH, workspace=ws)),
        )
        row = {}
        for name, f in cases:
            def run():
                for i in range(reps):
                    f(i)
            ms, _ = graph_time_ms(torch, run, replays=3, steady_ms=100.0)
            row[name] = round(ms * 1e3 / reps, 2)
        res["M=%d" % M] = row
    # the codes GEMVs over the token count: the part of a launch that grows with M
    sweep = {}
    for M in (1, 2, 4, 8, 12, 16):
        xq, xs = bl.quantize_acts(torch.randn((M, H), device=dev, generator=gen).to(torch.bfloat16))
        uq, us = bl.quantize_acts(torch.randn((M, F), device=dev, generator=gen).to(torch.bfloat16))
        yF = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        yH = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        for name, f in (("up", lambda i: bl.forward(xq, xs, *w_fh[i % copies], out=yF, workspace=ws)),
                        ("down", lambda i: bl.forward(uq, us, *w_hf[i % copies], out=yH, workspace=ws))):
            def run():
                for i in range(reps):
                    f(i)
            ms, _ = graph_time_ms(torch, run, replays=3, steady_ms=100.0)
            sweep.setdefault(name, {})["M=%d" % M] = round(ms * 1e3 / reps, 2)
    res["codes_gemv_by_tokens"] = sweep
    return res


def leg_parity_layer(torch, bl, reps=200):
    """The parity configuration timed (no roofline claim: 32 KB of weights): the single
    fp32 BitLinear at M=8, K=256, N=512, fused quantize + forward + ReLU^2, fp32 Y, for
    int8 / int4 codes and per-token / per-tensor scales."""
    import workloads
    dev = torch.device("cuda:0")
    W, X = workloads.parity_layer(seed=0, m=8, k=256, n=512)
    packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(dev))
    Xd = torch.from_numpy(X).to(dev)
    y = torch.empty((8, 512), dtype=torch.float32, device=dev)
    out = {"M": 8, "K": 256, "N": 512}
    for bits in (8, 4):
        for gran in ("token", "tensor"):
            ws = torch.empty(max(256, bl.workspace_size(bl.BL_OP_FORWARD_FUSED, 8, 512, 256, bits, gran)),
                             dtype=torch.uint8, device=dev)

            def run():
                for _ in range(reps):
                    bl.forward_fused(Xd, packed, gamma, bits=bits, gran=gran, epilogue="relu2", out=y,
                                     workspace=ws)
            ms = graph_time_ms(torch, run, replays=1)[0] / reps
            out["int%d_%s_us" % (bits, gran)] = ms * 1e3
    return out


def leg_backward(torch, bl, reps=5):
    """Backward pass under the straight-through estimators (bitlinear_backward: dX, dW and
    dbias from a bf16 dY), at the 2B prefill shapes (M=2048, int8 per-token codes, the
    b1.58 training layer) and at the 70B-class layer with 4-bit codes and both clipping
    masks (the a4.8 training layer).  Per shape: the whole call, dX alone and dW alone
    (each with its operand preparation).  Algorithmic flops: 2 M N K per gradient GEMM;
    per-token dW runs three bf16 passes (the fp32 operand in three exact parts), so the
    matrix cores execute 3x its algorithmic flops."""
    import workloads
    dev = torch.device("cuda:0")
    out = {}
    cases = [("up_2b", workloads.SHAPE_UP, 2048, 8, None),
             ("down_2b", workloads.SHAPE_DOWN, 2048, 8, None),
             ("layer_70b_int4", workloads.SHAPE_70B, 4096, 4, "masks")]
    for name, (K, N), M, bits, masks in cases:
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        W = (0.02 * torch.randn((N, K), device=dev, generator=gen))
        packed, gamma = bl.quantize_weights(W)
        X = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
        xq, s = bl.quantize_acts(X, bits=bits)
        dY = (0.01 * torch.randn((M, N), device=dev, generator=gen)).to(torch.bfloat16)
        Wb = W.to(torch.bfloat16) if masks else None
        del W
        Xm = X if masks else None
        ws = torch.empty(bl.workspace_size(bl.BL_OP_BACKWARD, M, N, K, bits), dtype=torch.uint8,
                         device=dev)
        res = {k: torch.empty(v, dtype=torch.float32, device=dev)
               for k, v in (("dX", (M, K)), ("dW", (N, K)), ("dbias", (N,)))}
        flops = 2.0 * M * N * K
        r = {"M": M, "K": K, "N": N, "bits": bits, "masks": bool(masks)}
        for tag, want in (("all", ("dX", "dW", "dbias")), ("dX", ("dX",)), ("dW", ("dW",))):
            def run():
                for _ in range(reps):
                    bl.backward(dY, xq, s, packed, gamma, bits=bits, X=Xm, W=Wb, want=want,
                                workspace=ws, out=res)
            ms = graph_time_ms(torch, run, replays=1)[0] / reps
            fl = flops * (2 if tag == "all" else 1)
            r[tag + "_us"] = ms * 1e3
            r[tag + "_tflops"] = fl / (ms * 1e-3) / 1e12
        r["dX_frac"] = r["dX_tflops"] / BF16_PEAK_TFLOPS
        # dW against its algorithmic flops (2 M N K), and against the work the matrix
        # cores execute (per-token scales: three bf16 passes, 3x)
        r["dW_frac"] = r["dW_tflops"] / BF16_PEAK_TFLOPS
        r["dW_mfma_tflops"] = 3 * r["dW_tflops"]  # every case here has per-token scales
        r["dW_mfma_frac"] = r["dW_mfma_tflops"] / BF16_PEAK_TFLOPS
        out[name] = r
        del packed, X, xq, dY, Wb, ws, res
        torch.cuda.synchronize()
    out["peak_tflops"] = BF16_PEAK_TFLOPS
    out["mfma"] = "bf16 32x32x16, fp32 accumulation, exact operands"
    return out


def leg_pack(torch, bl, reps=10):
    """a1: weight quantization + packing of the 2B up projection, fp32 W in HBM."""
    import workloads
    dev = torch.device("cuda:0")
    W, _ = workloads.decode_gemv(seed=1, shape=workloads.SHAPE_UP)
    Wd = torch.from_numpy(W).to(dev)
    packed, gamma = bl.quantize_weights(Wd)
    ws = torch.empty(bl.workspace_size(bl.BL_OP_QUANTIZE_WEIGHTS, 1, *W.shape), dtype=torch.uint8,
                     device=dev)

    def run():
        for _ in range(reps):
            bl.quantize_weights(Wd, workspace=ws, out=(packed, gamma))

    ms, _ = graph_time_ms(torch, run, replays=1)
    ms /= reps
    N, K = W.shape
    alg = 2 * 4 * N * K + N * K // 4  # two passes over fp32 W, packed write
    return {"N": N, "K": K, "us": ms * 1e3, "gbs": alg / (ms * 1e-3) / 1e9,
            "alg_bytes": alg}


def leg_acts(torch, bl, reps=20):
    """a2: per-token absmax activation quantization of bf16 X in HBM, at the prefill
    shapes (2B: M=2048, K=2560 and 6912; 70B: M=4096, K=8192), int8 and int4 codes.
    Algorithmic bytes: X read once (2MK), codes (MK or MK/2) and scales (4M) written."""
    dev = torch.device("cuda:0")
    out = {}
    for M, K in ((2048, 2560), (2048, 6912), (4096, 8192)):
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        # two copies alternate, so the 67 MB of the 70B input is not read from the
        # Infinity Cache on consecutive calls
        Xs = [torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16) for _ in range(2)]
        for bits in (8, 4):
            xq = torch.empty((M, K if bits == 8 else K // 2), dtype=torch.int8, device=dev)
            sc = torch.empty((M,), dtype=torch.float32, device=dev)

            def run():
                for i in range(reps):
                    bl.quantize_acts(Xs[i % 2], bits=bits, out=(xq, sc))

            ms, _ = graph_time_ms(torch, run, replays=1)
            ms /= reps
            alg = 2 * M * K + (M * K if bits == 8 else M * K // 2) + 4 * M
            out["%dx%d_int%d" % (M, K, bits)] = {
                "us": round(ms * 1e3, 2), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": alg}
        del Xs
    return out


CALIB_LIB = os.path.join(ROOT, "ternary_weight_quantized_bitlinear_amd", "libbitlinear_calib.so")


def leg_mfma_ceiling(torch, reps=3):
    """Matrix-core ceilings on this chip: MFMA-only loops (no memory, barrier or VALU work)
    on register operands with the value statistics of the int8 GEMMs (on both int8
    instruction shapes), the FP4 x FP6 GEMM and the backward's bf16 GEMMs
    (libbitlinear_calib.so), one 8-wave block per CU.
    Median of `reps` launches of a few ms each."""
    import ctypes
    lib = ctypes.CDLL(CALIB_LIB)
    lib.bl_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.bl_calib_mfma.restype = ctypes.c_int
    lib.bl_calib_ops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.bl_calib_ops.restype = ctypes.c_double
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    out = {"blocks": blocks, "waves_per_block": 8}
    for kind, name, iters, peak in ((0, "int8_32x32x32", 20000, INT8_PEAK_TOPS),
                                    (3, "int8_16x16x64", 40000, INT8_PEAK_TOPS),
                                    (1, "fp4_x_fp6_32x32x64", 10000, F6F4_PEAK_TOPS),
                                    (4, "fp4_x_fp6_16x16x128", 20000, F6F4_PEAK_TOPS),
                                    (2, "bf16_32x32x16", 20000, BF16_PEAK_TFLOPS)):
        def launch():
            st = lib.bl_calib_mfma(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError("calibration launch failed: HIP status %d" % st)
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        tops = lib.bl_calib_ops(kind, blocks, iters) / (ms * 1e-3) / 1e12
        out[name] = {"tops": round(tops, 1), "of_peak": round(tops / peak, 4), "ms": round(ms, 3)}
    return out


def leg_hbm_ceiling(torch, reps=5, mib=1024):
    """HBM read ceiling on this chip: a read-only sweep of 16-byte non-temporal loads over
    a buffer four times the last-level cache (libbitlinear_calib.so), at several grid
    sizes; the best median.  The weight-streaming decode kernels read and barely write,
    so this is the rate their fraction can be read against, beside the published peak."""
    import ctypes
    lib = ctypes.CDLL(CALIB_LIB)
    lib.bl_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.bl_calib_read.restype = ctypes.c_int
    nbytes = mib << 20
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    best = None
    sweep = {}
    modes = {0: "nt4", 1: "nt8", 2: "plain8"}
    for mode, blocks in [(m, b) for m in modes for b in (2048, 4096, 8192, 16384, 32768)]:
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

        def launch():
            st = lib.bl_calib_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, mode,
                                   ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError("calibration launch failed: HIP status %d" % st)
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        gbs = nbytes / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e9
        sweep["%s_%d" % (modes[mode], blocks)] = round(gbs, 1)
        if best is None or gbs > best[0]:
            best = (gbs, modes[mode], blocks)
    del buf
    return {"gbs": round(best[0], 1), "of_peak": round(best[0] / HBM_PEAK_GBS, 4),
            "loads": best[1], "blocks": best[2], "bytes": nbytes, "gbs_by_config": sweep}


def _timed(fn, budget_s, max_n=1000):
    """Calls fn() until budget_s of wall time has passed: (calls, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s or n >= max_n:
            return n, el


def cpu_baseline(x, W_up, W_dn, decode_budget_s=6.0):
    """The oracle (single-threaded C, as it stands: never tuned) timed on this host, pinned
    to one core for the duration, beside each configuration.  The headline entry is the
    same decode FFN step as the GPU's headline (GB/s of weights); the others time the
    oracle on the parity layer in full, and on bounded samples of the prefill GEMM, the
    30-layer stack and the 70B layer, extrapolated to the whole configuration and
    labelled as such.  A baseline for context, not a target."""
    import oracle
    import workloads
    before = os.sched_getaffinity(0)
    core = min(before)
    os.sched_setaffinity(0, {core})
    try:
        host = {"cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
                "cpus_allowed_before_pinning": len(before), "pinned_to_cpu": core}
        # C2: the decode FFN step (the headline's unit)
        p_up, g_up, _ = oracle.quantize_weights(W_up)
        p_dn, g_dn, _ = oracle.quantize_weights(W_dn)
        (K1, N1), (K2, N2) = workloads.SHAPE_UP, workloads.SHAPE_DOWN

        def step():
            h, _, _, _ = oracle.bitlinear(x, p_up, g_up, epi=oracle.EPI_RELU2, y_dtype=oracle.BF16)
            oracle.bitlinear(h, p_dn, g_dn, y_dtype=oracle.BF16)
        n, el = _timed(step, decode_budget_s, 5000)
        step_bytes = gemv_bytes(K1, N1) + gemv_bytes(K2, N2)
        out = {"value": step_bytes * n / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "%d decode FFN steps (up 2560->6912 + ReLU^2, down 6912->2560, M=1, "
                         "int8 per token, bf16 out) in %.1f s on one core of %s" % (
                             n, el, host["cpu_model"]),
               "ms_per_step": el * 1e3 / n, **host}
        per = {}
        # C1: the parity layer, whole (weights, activations, forward with ReLU^2)
        W, X = workloads.parity_layer(seed=0, m=8, k=256, n=512)

        def c1():
            pk, g, _ = oracle.quantize_weights(W)
            oracle.bitlinear(X, pk, g, epi=oracle.EPI_RELU2)
        n, el = _timed(c1, 1.5)
        per["c1_parity_layer"] = {"us_per_call": el * 1e6 / n, "calls": n,
                                  "sample": "whole call: quantize W 512x256, quantize X 8x256, "
                                            "forward + ReLU^2, fp32 out"}
        # C3: the prefill up projection, 16 of its 2048 token rows, all outputs
        W3, X3 = workloads.prefill_gemm(seed=2, shape=workloads.SHAPE_UP)
        p3, g3, _ = oracle.quantize_weights(W3)
        rows = X3[:16]
        t0 = time.perf_counter()
        oracle.bitlinear(rows, p3, g3, epi=oracle.EPI_RELU2, y_dtype=oracle.BF16)
        el = time.perf_counter() - t0
        K, N = workloads.SHAPE_UP
        full_s = el * 2048 / 16
        per["c3_prefill_up"] = {"s_extrapolated": full_s,
                                "tops_extrapolated": 2.0 * 2048 * N * K / full_s / 1e12,
                                "sample": "16 of 2048 token rows x all 6912 outputs in %.2f s, "
                                          "extrapolated linearly to M=2048" % el}
        # C4: one block of the batch-16 stack (norm, QKV, O, norm, up + ReLU^2, down)
        codes = workloads.stack_layer_codes(3, 0)
        lw = {k: oracle.quantize_weights(c.astype(np.float32))[:2] for k, c in codes.items()}
        x0 = workloads.stack_input(seed=3, m=16)
        H = workloads.HIDDEN
        t0 = time.perf_counter()
        x1, h1 = oracle.rmsnorm(x0)
        q1, s1 = oracle.quantize_acts(h1)
        pq, gq = lw["qkv"]
        for part in range(3):
            y, _ = oracle.forward(q1, 8, s1, oracle.PER_TOKEN, pq[part * H:(part + 1) * H], gq,
                                  y_dtype=oracle.BF16)
        o, _, _, _ = oracle.bitlinear(y, *lw["o"], y_dtype=oracle.BF16)
        x2, h2 = oracle.rmsnorm(x1, o)
        u, _, _, _ = oracle.bitlinear(h2, *lw["up"], epi=oracle.EPI_RELU2, y_dtype=oracle.BF16)
        oracle.bitlinear(u, *lw["down"], y_dtype=oracle.BF16)
        el = time.perf_counter() - t0
        per["c4_stack_2b"] = {"ms_per_step_extrapolated": el * 1e3 * workloads.LAYERS_2B,
                              "tokens_per_s_extrapolated": 16 / (el * workloads.LAYERS_2B),
                              "sample": "layer 0 of 30 at batch 16 in %.2f s, times 30" % el}
        # C5: the 70B layer with int4 activations, 4 of its 4096 token rows
        c5codes, X5 = workloads.layer_70b(m=4)
        p5, g5, _ = oracle.quantize_weights(c5codes.astype(np.float32))
        del c5codes
        t0 = time.perf_counter()
        oracle.bitlinear(X5, p5, g5, bits=4, y_dtype=oracle.BF16)
        el = time.perf_counter() - t0
        K5, N5 = workloads.SHAPE_70B
        full_s = el * 4096 / 4
        per["c5_70b_int4"] = {"s_extrapolated": full_s,
                              "tops_extrapolated": 2.0 * 4096 * N5 * K5 / full_s / 1e12,
                              "sample": "4 of 4096 token rows x all 28672 outputs in %.2f s, "
                                        "extrapolated linearly to M=4096" % el}
        out["per_config"] = per
        return out
    finally:
        os.sched_setaffinity(0, before)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=64, help="layers per streamed launch")
    ap.add_argument("--copies", type=int, default=64, help="weight copies of the chain leg")
    ap.add_argument("--chain-steps", type=int, default=2000)
    ap.add_argument("--legs", default="decode,chain,single,c1,prefill,stack,c5,pack,acts,backward,"
                                      "ceiling,cpu")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import ternary_weight_quantized_bitlinear_amd as bl
    if not os.path.exists(bl.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    legs = set(args.legs.split(","))
    if "traffic" in legs:
        leg_traffic(torch, bl)
    if "decode" not in legs:
        # counter runs: only the named legs, no headline line
        side = {}
        if "prefill" in legs:
            side["prefill"] = leg_prefill(torch, bl)
        if "pack" in legs:
            side["pack"] = leg_pack(torch, bl)
        if "acts" in legs:
            side["acts"] = leg_acts(torch, bl)
        if "c5" in legs:
            side["layer_70b"] = leg_70b(torch, bl)
        if "stack" in legs:
            side["stack_2b"] = leg_stack(torch, bl)
        if "backward" in legs:
            side["backward"] = leg_backward(torch, bl)
        if "c1" in legs:
            side["parity_layer"] = leg_parity_layer(torch, bl)
        if "ceiling" in legs:
            side["mfma_ceiling"] = leg_mfma_ceiling(torch)
            side["hbm_read_ceiling"] = leg_hbm_ceiling(torch)
        if "launches" in legs:
            side["stack_launches_us"] = leg_stack_launches(torch, bl)
        if side:
            print(json.dumps(side))
        return

    st = leg_decode_stream(torch, bl, args.steps, args.warmup, args.batch)
    alg = st["bytes_per_launch"] / (st["per_launch_us"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(st["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "arithmetic": "int8 x ternary -> int32 accumulation, fp32 rescale, bf16 in and out",
        "data": "synthetic: seeded uniform-ternary weights, N(0,1) bf16 activations",
        "config": {"workload": "BitNet-2B FFN decode GEMVs, M=1, streamed: %d independent layers "
                               "per launch; step = up 2560->6912 (+ReLU^2) then down 6912->2560 "
                               "on every layer, fused int8 per-token quantization, bf16 out; "
                               "steps cycle %d weight sets (%d MB) so weights come from HBM"
                               % (st["batch"], st["sets"], st["sets"] * st["step_bytes"] // 10**6),
                   "weight_sets": st["sets"],
                   "tokens_per_layer": 1, "hidden": 2560, "ffn": 6912,
                   "layers_per_launch": st["batch"], "weight_bytes_per_step": st["step_bytes"]},
        "roofline": {"bound": "hbm", "kernel": "gemv_stream_kernel (fused decode GEMV, 64 layers per launch)",
                     "achieved": round(alg, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "bytes_per_launch": st["bytes_per_launch"],
                     "us_per_launch": st["per_launch_us"],
                     "repeat_us_per_launch": [round(v * 1e3 / 2, 2)
                                              for v in st["repeat_ms_per_step"]]},
    }
    if "chain" in legs:
        dec = leg_decode(torch, bl, args.chain_steps, args.warmup, args.copies)
        out["decode_chain"] = {
            "workload": "one 2B FFN decode step, M=1, single layer: up (+ReLU^2) then down, two "
                        "dependent launches; %d weight copies rotated (%d B)" % (
                            dec["weight_copies"], dec["rotation_bytes"]),
            "us_per_step": dec["ms_per_step"] * 1e3, "gbs": round(dec["gbs"], 2),
            "frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
            "us_per_launch": dec["per_launch_us"]}
    if "single" in legs:
        out["decode_single"] = leg_decode_single(torch, bl)
    if "prefill" in legs:
        pf = leg_prefill(torch, bl)
        out["prefill"] = {"metric": "prefill GEMM int TOPS (2*M*N*K / GEMM time)",
                          "workload": "M=2048 tokens, 2560->6912 (+ReLU^2) and 6912->2560, "
                                      "int8 per token, bf16 out",
                          "value": round(pf["gemm_tops"], 2), "unit": "TOPS",
                          "mfma": "int8 16x16x64 in balanced tiles: 128 x 448 (up), 128 x 160 "
                                  "(down)",
                          "roofline": {"bound": "mfma", "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                                       "frac": round(pf["gemm_frac"], 4)},
                          "with_act_quant_tops": round(pf["step_tops"], 2),
                          "shapes": {k: pf[k] for k in ("up", "down")},
                          "int4_activations": pf["int4"]}
    if "pack" in legs:
        out["pack"] = leg_pack(torch, bl)
    if "acts" in legs:
        out["acts"] = {"workload": "per-token absmax quantization of bf16 X (a2), prefill shapes",
                       "unit": "GB/s", "peak": HBM_PEAK_GBS, **leg_acts(torch, bl)}
    if "stack" in legs:
        out["stack_2b"] = {"workload": "30-layer BitNet-2B-shaped decode stack, batch 16: QKV, O, "
                                       "up (+ReLU^2), down per layer with RMS norm, residual and "
                                       "requantization between them",
                           **leg_stack(torch, bl)}
    if "c5" in legs:
        c5 = leg_70b(torch, bl)
        out["layer_70b"] = {"workload": "70B-class FFN layer, M=4096 tokens, K=8192, N=28672, "
                                        "0.5% outlier channels x30, bf16 out: int8 vs int4 "
                                        "activations",
                            "unit": "TOPS", "peak_int8": INT8_PEAK_TOPS, **c5}
    if "c1" in legs:
        out["parity_layer"] = {"workload": "single fp32 BitLinear, M=8, K=256, N=512, fused "
                                           "quantize + forward + ReLU^2, fp32 out (timed only)",
                               **leg_parity_layer(torch, bl)}
    if "backward" in legs:
        out["backward"] = {"workload": "straight-through-estimator backward (dX, dW, dbias from "
                                       "bf16 dY): 2B FFN shapes at M=2048 with int8 codes, and "
                                       "the 70B-class layer at M=4096 with int4 codes and both "
                                       "clipping masks",
                           "unit": "TFLOP/s", **leg_backward(torch, bl)}
    if "ceiling" in legs:
        # each matrix-core rate beside the MFMA-only ceiling measured for its operands
        ceil = leg_mfma_ceiling(torch)
        out["mfma_ceiling"] = ceil
        hbm = leg_hbm_ceiling(torch)
        out["hbm_read_ceiling"] = hbm
        out["roofline"]["read_ceiling_gbs"] = hbm["gbs"]
        out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / hbm["gbs"], 4)
        c8m = ceil["int8_16x16x64"]["tops"]
        c4 = ceil["fp4_x_fp6_32x32x64"]["tops"]
        cb = ceil["bf16_32x32x16"]["tops"]
        if "prefill" in out:
            # the 2B prefill shapes and the 70B layer run on the 16x16x64 int8 matrix cores
            pf = out["prefill"]
            pf["roofline"]["mfma_ceiling_tops"] = c8m
            pf["roofline"]["frac_of_ceiling"] = round(pf["value"] / c8m, 4)
            pf["int4_activations"]["frac_of_ceiling"] = round(
                pf["int4_activations"]["gemm_tops"] / c4, 4)
        if "layer_70b" in out:
            l7 = out["layer_70b"]
            l7["int8"]["frac_of_ceiling"] = round(l7["int8"]["gemm_tops"] / c8m, 4)
            l7["int4"]["frac_of_ceiling"] = round(l7["int4"]["gemm_tops"] / c4, 4)
        if "backward" in out:
            for k, r in out["backward"].items():
                if isinstance(r, dict) and "dX_tflops" in r:
                    r["dX_frac_of_ceiling"] = round(r["dX_tflops"] / cb, 4)
                    r["dW_mfma_frac_of_ceiling"] = round(r["dW_mfma_tflops"] / cb, 4)
    if "cpu" in legs:
        out["cpu_baseline"] = cpu_baseline(st["x"], st["W_up"], st["W_dn"])
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
