"""Seeded synthetic inputs for the ZETA causal top-k attention path.

This module only draws random numbers; it contains none of the method's arithmetic
(no quantisation, no interleaving, no selection, no weighting).  Both the CPU oracle tests
and the GPU path take their inputs from here, so the two sides see identical bytes.

Recipe (numpy PCG64 via ``default_rng(seed)``; draw order q, k, v, gamma, dout):

* ``normal``    -- q, k ~ N(0, 1) per coordinate, float64 draws cast to fp32.
* ``clustered`` -- per (b, h) 16 centres ~ U[-3, 3]^3; every q and every k token picks a
                   centre uniformly and adds N(0, 0.05^2 I).  Many tokens then share a
                   Z-order cell, which exercises the tie rule.
* ``discrete``  -- every coordinate drawn from a small fixed set of values, so that codes
                   collide heavily (tie-heavy test inputs).
* v, dout ~ N(0, 1) drawn directly in fp32; bf16 values are the round-to-nearest-even of
  the fp32 draw and are carried as raw uint16 bit patterns.
* gamma: a fixed value, or U[0.5, 2.0] per head.
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, distributions and seed."""

    name: str
    B: int
    H: int
    N: int
    dv: int
    topk: int
    v_dtype: str = F32
    dist: str = "normal"
    gamma: float | None = None  # fixed value, or None for U[0.5, 2.0] per head
    seed: int = 0
    backward: bool = False

    @property
    def rows(self) -> int:
        return self.B * self.H * self.N


# The five workloads the pages' causal setting is measured on (sizes of the
# 65536-token efficiency point in the "Measured effects" table of the paper summary page,
# plus smaller multi-head and clustered cases).
CONFIGS = {
    "tiny": Workload("tiny", 1, 1, 1024, 64, 32, F32, "normal", 1.0, seed=1),
    "multihead": Workload("multihead", 1, 8, 4096, 64, 32, F32, "normal", None, seed=2),
    "clustered": Workload("clustered", 4, 8, 16384, 64, 64, F32, "clustered", None, seed=3),
    "long_fwd": Workload("long_fwd", 1, 8, 65536, 128, 32, BF16, "normal", None, seed=4),
    "long_fwd_bwd": Workload("long_fwd_bwd", 1, 8, 65536, 128, 32, BF16, "normal", None,
                             seed=4, backward=True),
}

DISCRETE_VALUES = np.array([-1.0, -0.25, 0.0, 0.5, 2.0], dtype=np.float64)


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); uint16 bit patterns.

    uint32 arithmetic cannot overflow here: finite fp32 bit patterns are at most
    0xFF7FFFFF, so adding at most 0x8000 stays below 2^32."""
    b = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = b >> 16
    lsb &= 1
    b += 0x7FFF
    b += lsb
    b >>= 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _qk(rng: np.random.Generator, w: Workload) -> tuple[np.ndarray, np.ndarray]:
    shape = (w.B, w.H, w.N, 3)
    if w.dist == "normal":
        q = rng.standard_normal(shape)
        k = rng.standard_normal(shape)
    elif w.dist == "clustered":
        centres = rng.uniform(-3.0, 3.0, size=(w.B, w.H, 16, 3))
        bi = np.arange(w.B)[:, None, None]
        hi = np.arange(w.H)[None, :, None]
        qa = rng.integers(0, 16, size=(w.B, w.H, w.N))
        q = centres[bi, hi, qa] + 0.05 * rng.standard_normal(shape)
        ka = rng.integers(0, 16, size=(w.B, w.H, w.N))
        k = centres[bi, hi, ka] + 0.05 * rng.standard_normal(shape)
    elif w.dist == "discrete":
        q = DISCRETE_VALUES[rng.integers(0, len(DISCRETE_VALUES), size=shape)]
        k = DISCRETE_VALUES[rng.integers(0, len(DISCRETE_VALUES), size=shape)]
    elif w.dist == "constant":
        q = np.full(shape, 0.3)
        k = np.full(shape, 0.3)
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    return q.astype(np.float32), k.astype(np.float32)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == BF16:
        return fp32_to_bf16_bits(x)
    if dtype == F32:
        return x
    raise ValueError(f"unknown value dtype {dtype!r}")


def make_inputs(w: Workload) -> dict:
    """Draw the inputs of workload ``w``; arrays are C-contiguous numpy arrays.

    Returns q, k (fp32 [B,H,N,3]), v ([B,H,N,dv], fp32 or bf16 bits), gamma (fp32 [H]) and,
    for backward workloads, dout (same layout and dtype as v).
    """
    rng = np.random.default_rng(w.seed)
    q, k = _qk(rng, w)
    v = _values(rng, (w.B, w.H, w.N, w.dv), w.v_dtype)
    if w.gamma is None:
        gamma = rng.uniform(0.5, 2.0, size=w.H).astype(np.float32)
    else:
        gamma = np.full(w.H, w.gamma, dtype=np.float32)
    out = {"q": q, "k": k, "v": v, "gamma": gamma}
    if w.backward:
        out["dout"] = _values(rng, (w.B, w.H, w.N, w.dv), w.v_dtype)
    return out


def digest(arrays: dict) -> str:
    """SHA-256 over the input arrays in a fixed key order (logged next to results)."""
    h = hashlib.sha256()
    for key in sorted(arrays):
        h.update(key.encode())
        h.update(np.ascontiguousarray(arrays[key]).tobytes())
    return h.hexdigest()
