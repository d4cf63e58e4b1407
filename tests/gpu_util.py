"""Helpers shared by the GPU parity tests: host <-> device transfer of the seeded
inputs, and element-by-element comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    """Name the case before each GPU step (flushed), so a failure points at it."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_same_bytes(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g = got.view(np.uint8).reshape(-1)
    r = ref.view(np.uint8).reshape(-1)
    bad = np.nonzero(g != r)[0]
    assert bad.size == 0, "%s: %d of %d bytes differ, first at byte %d (got %d, ref %d)" % (
        what, bad.size, g.size, bad[0], g[bad[0]], r[bad[0]])


def assert_y_matches(got: np.ndarray, ref: np.ndarray, y_dtype: str, what: str):
    """Outputs: within 1e-5 relative in fp32 (exact zeros stay zeros), and within one bf16
    ulp for bf16 -- then bit-identical, which the fixed fp32 operation order promises."""
    if y_dtype == "f32":
        g = got.astype(np.float64)
        r = ref.astype(np.float64)
        err = np.abs(g - r)
        tol = 1e-5 * np.abs(r)
        bad = err > tol
        assert not bad.any(), "%s: %d outputs beyond 1e-5 relative (max rel %.3g)" % (
            what, int(bad.sum()), float((err / np.maximum(np.abs(r), 1e-30)).max()))
        assert_same_bytes(got.astype(np.float32), ref.astype(np.float32), what + " (bits)")
    elif y_dtype == "bf16":
        d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
        assert d.max(initial=0) <= 1, "%s: bf16 outputs more than one ulp apart" % what
        assert_same_bytes(got, ref, what + " (bits)")
    else:
        assert_same_bytes(got, ref, what)


def sample_positions(M: int, N: int, count: int, seed: int = 0):
    """Random (m, n) positions plus every corner, one full row and one full column."""
    rng = np.random.default_rng(seed)
    ms = [rng.integers(0, M, count)]
    ns = [rng.integers(0, N, count)]
    corners = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    ms.append(np.array([c[0] for c in corners]))
    ns.append(np.array([c[1] for c in corners]))
    r = int(rng.integers(0, M))
    ms.append(np.full(N, r))
    ns.append(np.arange(N))
    c = int(rng.integers(0, N))
    ms.append(np.arange(M))
    ns.append(np.full(M, c))
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)
