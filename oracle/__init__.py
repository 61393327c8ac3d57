"""CPU oracle for ZETA causal top-k attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 definition of what the GPU path computes (``zeta_oracle.c``, built with
gcc into ``liboracle.so``).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path never does.
It shares no code with the HIP path.

Parity pins: see ``tests/test_oracle_pins.py`` (hand-worked codes and cells, closed forms,
invariants, finite differences and a dense library special case).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zeta_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_cell.argtypes = [ctypes.c_float]
        lib.oracle_cell.restype = ctypes.c_int32
        lib.oracle_interleave.argtypes = [ctypes.c_int32] * 3
        lib.oracle_interleave.restype = ctypes.c_uint32
        lib.oracle_encode.argtypes = [p, i64, p]
        lib.oracle_select_codes.argtypes = [i64, i64, p, p, i64, p, p]
        lib.oracle_select.argtypes = [i64, i64, i64, p, p, i64, p, p]
        lib.oracle_forward.argtypes = [i64, i64, i64, i64, ctypes.c_int, p, p, p, p, i64, p,
                                       p, p, p]
        lib.oracle_backward.argtypes = [i64, i64, i64, i64, ctypes.c_int, p, p, p, p, p, i64,
                                        p, p, p, p, p, p]
        lib.oracle_cell12.argtypes = [ctypes.c_float]
        lib.oracle_cell12.restype = ctypes.c_int32
        lib.oracle_interleave36.argtypes = [ctypes.c_int32] * 3
        lib.oracle_interleave36.restype = ctypes.c_uint64
        lib.oracle_encode_ex.argtypes = [p, i64, ctypes.c_int, p, p]
        lib.oracle_select_codes64.argtypes = [i64, i64, ctypes.c_int, p, p, i64, p, p]
        lib.oracle_chunk_len.argtypes = [i64, i64]
        lib.oracle_chunk_len.restype = i64
        lib.oracle_select_chunked.argtypes = [i64, i64, i64, p, p, i64, p, p]
        lib.oracle_select_multi.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, p, p,
                                            i64, p, p]
        lib.oracle_euclid_topk.argtypes = [i64, i64, ctypes.c_int, p, p, i64, p, p]
        lib.oracle_bf16_bits.argtypes = [ctypes.c_double]
        lib.oracle_bf16_bits.restype = ctypes.c_uint16
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return _load().oracle_max_threads()


def cell(x: float) -> int:
    return int(_load().oracle_cell(float(x)))


def interleave(c0: int, c1: int, c2: int) -> int:
    return int(_load().oracle_interleave(c0, c1, c2))


def encode(x: np.ndarray) -> np.ndarray:
    """Z-order codes (uint32) of fp32 points [..., 3]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.size // 3
    z = np.empty(x.shape[:-1], dtype=np.uint32)
    _load().oracle_encode(_ptr(x), rows, _ptr(z))
    return z


def _rows(rows, total: int) -> np.ndarray:
    if rows is None:
        return np.arange(total, dtype=np.int64)
    return np.ascontiguousarray(rows, dtype=np.int64)


def select_codes(zq: np.ndarray, zk: np.ndarray, N: int, topk: int, rows=None) -> np.ndarray:
    """Exact causal top-k by (|zq-zk|, j) from codes; idx [len(rows), topk], -1 padded."""
    zq = np.ascontiguousarray(zq, dtype=np.uint32).reshape(-1)
    zk = np.ascontiguousarray(zk, dtype=np.uint32).reshape(-1)
    r = _rows(rows, zq.size)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_select_codes(N, topk, _ptr(zq), _ptr(zk), r.size, _ptr(r), _ptr(idx))
    return idx


def select(q: np.ndarray, k: np.ndarray, topk: int, rows=None) -> np.ndarray:
    """Exact causal top-k from fp32 points q, k [B,H,N,3]; idx [len(rows), topk]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    B, H, N, _ = q.shape
    r = _rows(rows, B * H * N)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_select(B * H, N, topk, _ptr(q), _ptr(k), r.size, _ptr(r), _ptr(idx))
    return idx


def cell12(x: float) -> int:
    return int(_load().oracle_cell12(float(x)))


def interleave36(c0: int, c1: int, c2: int) -> int:
    return int(_load().oracle_interleave36(c0, c1, c2))


def encode_ex(x: np.ndarray, bits: int = 10, perm=(0, 1, 2)) -> np.ndarray:
    """Z-order codes (uint64) with `bits` (10 or 12) per axis, axis a from coordinate perm[a]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    z = np.empty(x.shape[:-1], dtype=np.uint64)
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    _load().oracle_encode_ex(_ptr(x), x.size // 3, int(bits), _ptr(pm), _ptr(z))
    return z


def select_codes64(zq, zk, N: int, topk: int, causal: bool = True, rows=None) -> np.ndarray:
    """Exact top-k by (|zq-zk|, j) over uint64 codes, causal (j <= i) or not (j < N)."""
    zq = np.ascontiguousarray(zq, dtype=np.uint64).reshape(-1)
    zk = np.ascontiguousarray(zk, dtype=np.uint64).reshape(-1)
    r = _rows(rows, zq.size)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_select_codes64(N, topk, int(causal), _ptr(zq), _ptr(zk), r.size, _ptr(r),
                                  _ptr(idx))
    return idx


def select_ex(q, k, topk: int, bits: int = 10, causal: bool = True, rows=None) -> np.ndarray:
    """Exact selection from fp32 points with `bits` per axis, causal or not."""
    N = q.shape[-2]
    return select_codes64(encode_ex(q, bits), encode_ex(k, bits), N, topk, causal, rows)


def chunk_len(N: int, chunks: int) -> int:
    return int(_load().oracle_chunk_len(N, chunks))


def select_chunked(zq, zk, N: int, topk: int, chunks: int, rows=None) -> np.ndarray:
    """The chunked causal search (window around the insertion position in each chunk) on
    10- or 12-bit codes."""
    zq = np.ascontiguousarray(zq, dtype=np.uint64).reshape(-1)
    zk = np.ascontiguousarray(zk, dtype=np.uint64).reshape(-1)
    r = _rows(rows, zq.size)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_select_chunked(N, topk, chunks, _ptr(zq), _ptr(zk), r.size, _ptr(r),
                                  _ptr(idx))
    return idx


def select_multi(q, k, topk: int, curves: int, causal: bool = True, rows=None,
                 bits: int = 10) -> np.ndarray:
    """Several curves (3 or 6 axis orders), each its own top-(topk // curves), merged."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    B, H, N, _ = q.shape
    r = _rows(rows, B * H * N)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_select_multi(B * H, N, topk, curves, int(causal), int(bits), _ptr(q), _ptr(k),
                                r.size, _ptr(r), _ptr(idx))
    return idx


def euclid_topk(q, k, topk: int, causal: bool = True, rows=None) -> np.ndarray:
    """Exact Euclidean top-k of the raw points by (d^2, j) (recall diagnostic)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    B, H, N, _ = q.shape
    r = _rows(rows, B * H * N)
    idx = np.empty((r.size, topk), dtype=np.int32)
    _load().oracle_euclid_topk(N, topk, int(causal), _ptr(q), _ptr(k), r.size, _ptr(r),
                               _ptr(idx))
    return idx


def forward(q, k, v, gamma, idx, v_bf16: bool, rows=None, want_weights: bool = False):
    """fp64 Cauchy-weighted output for the listed rows given their selection idx."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    B, H, N, _ = q.shape
    dv = v.shape[-1]
    r = _rows(rows, B * H * N)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(r.size, -1)
    K = idx.shape[1]
    out = np.empty((r.size, dv), dtype=np.float64)
    w = np.empty((r.size, K), dtype=np.float64) if want_weights else None
    _load().oracle_forward(H, N, K, dv, int(v_bf16), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                           r.size, _ptr(r), _ptr(idx), _ptr(out),
                           _ptr(w) if w is not None else None)
    return (out, w) if want_weights else out


def backward(q, k, v, gamma, dout, idx, v_bf16: bool, rows=None):
    """fp64 gradients with the selection fixed: (dq [rows,3], dk, dv, dgamma [H]).

    dk [B,H,N,3] and dv [B,H,N,dv] hold the contributions of the listed rows only."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v)
    dout = np.ascontiguousarray(dout)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    B, H, N, _ = q.shape
    dv = v.shape[-1]
    r = _rows(rows, B * H * N)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(r.size, -1)
    K = idx.shape[1]
    dq = np.empty((r.size, 3), dtype=np.float64)
    dk = np.zeros((B, H, N, 3), dtype=np.float64)
    dvv = np.zeros((B, H, N, dv), dtype=np.float64)
    dg = np.zeros(H, dtype=np.float64)
    _load().oracle_backward(H, N, K, dv, int(v_bf16), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                            _ptr(dout), r.size, _ptr(r), _ptr(idx), _ptr(dq), _ptr(dk),
                            _ptr(dvv), _ptr(dg))
    return dq, dk, dvv, dg


def bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 (nearest even), as uint16 bit patterns."""
    lib = _load()
    flat = np.asarray(x, dtype=np.float64).reshape(-1)
    out = np.fromiter((lib.oracle_bf16_bits(float(t)) for t in flat), dtype=np.uint16,
                      count=flat.size)
    return out.reshape(np.shape(x))
