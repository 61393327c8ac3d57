"""Helpers shared by the GPU parity tests: device transfer and the tolerance rule."""

from __future__ import annotations

import sys

import numpy as np
import torch

from order_retrieval_amd import inputs

# Tolerances of the floating-point outputs and gradients, by value dtype: max-abs error 1e-4
# when v is fp32 and 2e-2 when v is bf16.  bf16 outputs (o, dv) with |ref| >= 8 may also be
# off by one bf16 ulp of the reference, since at that size the rounding step alone exceeds
# 2e-2.  The oracle's fp64 result is the reference (not rounded).
ATOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def device_inputs(w: inputs.Workload, x: dict) -> dict:
    bf = w.v_dtype == inputs.BF16
    d = {"q": to_dev(x["q"]), "k": to_dev(x["k"]), "v": to_dev(x["v"], bf),
         "gamma": to_dev(x["gamma"])}
    if "dout" in x:
        d["dout"] = to_dev(x["dout"], bf)
    return d


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_close(gpu: np.ndarray, ref: np.ndarray, v_dtype: str, what: str,
                 bf16_output: bool = False) -> float:
    gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
    err = np.abs(gpu - ref)
    tol = np.full(ref.shape, ATOL[v_dtype])
    if bf16_output:
        tol = np.where(np.abs(ref) >= 8.0, np.maximum(tol, bf16_ulp(ref)), tol)
    bad = err > tol
    worst = float(err.max()) if err.size else 0.0
    log(f"  {what}: max|err| {worst:.3e} over {err.size} values (v {v_dtype})")
    if bad.any():
        pos = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} values beyond tolerance; worst at {pos}: "
                             f"gpu {gpu[pos]!r} ref {ref[pos]!r}")
    return worst


def sample_rows(w: inputs.Workload, count: int, seed: int = 0) -> np.ndarray:
    """Flat query rows to check at full size: random rows plus every head's first and last
    rows and rows just around power-of-two positions (where the run split changes)."""
    rng = np.random.default_rng(seed)
    BH, N = w.B * w.H, w.N
    picks = set(rng.integers(0, BH * N, size=count).tolist())
    for bh in {0, BH - 1}:
        for i in list(range(min(N, 70))) + list(range(max(0, N - 70), N)):
            picks.add(bh * N + i)
        p = 1
        while p < N:
            for i in (p - 2, p - 1, p, p + 1):
                if 0 <= i < N:
                    picks.add(bh * N + i)
            p *= 2
    return np.array(sorted(picks), dtype=np.int64)
