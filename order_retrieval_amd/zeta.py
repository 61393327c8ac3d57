"""Thin Python binding of ``libzeta.so`` (the C ABI of ``include/zeta.h``).

Argument marshalling only: every step of the path runs in the HIP kernels behind the C
ABI.  PyTorch provides device memory (outputs, workspaces) and the current HIP stream.
Loading fails loudly when the library has not been built; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzeta.so")

ZETA_OK = 0
ZETA_ERR_INVALID_ARGUMENT = 1
ZETA_ERR_UNSUPPORTED = 2
ZETA_ERR_WORKSPACE_TOO_SMALL = 3
ZETA_ERR_HIP = 4

ZETA_F32 = 0
ZETA_BF16 = 1

ZETA_WS_SELECT = 0
ZETA_WS_FWD = 1
ZETA_WS_BWD = 2

ZETA_MAX_TOPK = 256
ZETA_MAX_DV = 512
ZETA_MAX_CHUNKS = 1024

ZETA_SELECT_EXACT = 0
ZETA_SELECT_CHUNKED = 1
ZETA_SELECT_CURVES = 2

EXPORTS = (
    "zeta_workspace_bytes",
    "zeta_probe_row_gather",
    "zeta_fwd_noalloc",
    "zeta_encode",
    "zeta_tree_levels",
    "zeta_build_tree",
    "zeta_select",
    "zeta_fwd",
    "zeta_bwd",
    "zeta_workspace_bytes_ex",
    "zeta_select_ex",
    "zeta_fwd_ex",
    "zeta_bwd_ex",
    "zeta_set_stage_events",
    "zeta_status_string",
    "zeta_last_error",
)


class ZetaShape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("dv", ctypes.c_int64),
        ("topk", ctypes.c_int64),
        ("v_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class ZetaSelectOpts(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("chunks", ctypes.c_int32),
        ("curves", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def select_opts(mode: int = ZETA_SELECT_EXACT, causal: bool = True, bits: int = 10,
                chunks: int = 0, curves: int = 0) -> ZetaSelectOpts:
    return ZetaSelectOpts(mode, int(causal), bits, chunks, curves, 0)


def _opts_ref(opts: ZetaSelectOpts | None):
    return ctypes.byref(opts) if opts is not None else None


class ZetaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libzeta.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m order_retrieval_amd.build`")
    lib = ctypes.CDLL(path)
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime is mapped: {runtimes}")
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sp = ctypes.POINTER(ZetaShape)
    lib.zeta_workspace_bytes.argtypes = [sp, i32]
    lib.zeta_workspace_bytes.restype = sz
    lib.zeta_encode.argtypes = [p, i64, p, p]
    lib.zeta_encode.restype = i32
    lib.zeta_tree_levels.argtypes = [i64]
    lib.zeta_tree_levels.restype = i32
    lib.zeta_build_tree.argtypes = [i64, i64, p, p, p, p]
    lib.zeta_build_tree.restype = i32
    lib.zeta_select.argtypes = [sp, p, p, p, p, sz, p]
    lib.zeta_select.restype = i32
    op = ctypes.POINTER(ZetaSelectOpts)
    lib.zeta_workspace_bytes_ex.argtypes = [sp, op, i32]
    lib.zeta_workspace_bytes_ex.restype = sz
    lib.zeta_select_ex.argtypes = [sp, op, p, p, p, p, sz, p]
    lib.zeta_select_ex.restype = i32
    lib.zeta_fwd_ex.argtypes = [sp, op, p, p, p, p, p, p, p, sz, p]
    lib.zeta_fwd_ex.restype = i32
    lib.zeta_bwd_ex.argtypes = [sp, op, p, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.zeta_bwd_ex.restype = i32
    lib.zeta_fwd.argtypes = [sp, p, p, p, p, p, p, p, sz, p]
    lib.zeta_fwd.restype = i32
    lib.zeta_fwd_noalloc.argtypes = [sp, p, p, p, p, p, p, p]
    lib.zeta_fwd_noalloc.restype = i32
    lib.zeta_bwd.argtypes = [sp, p, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.zeta_bwd.restype = i32
    lib.zeta_probe_row_gather.argtypes = [p, i64, i32, i64, i32, ctypes.c_uint32, p, p]
    lib.zeta_probe_row_gather.restype = i32
    lib.zeta_set_stage_events.argtypes = [p, i32]
    lib.zeta_set_stage_events.restype = i32
    lib.zeta_status_string.argtypes = [i32]
    lib.zeta_status_string.restype = ctypes.c_char_p
    lib.zeta_last_error.argtypes = []
    lib.zeta_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def hip_runtimes_mapped() -> list[str]:
    """Files of libamdhip64 mapped into this process (torch's copy is shared with libzeta)."""
    with open("/proc/self/maps") as f:
        return sorted({line.split()[-1] for line in f if "libamdhip64" in line})


def _status_name(status: int) -> str:
    return load_library().zeta_status_string(status).decode()


def _check(status: int) -> None:
    if status != ZETA_OK:
        raise ZetaError(status, load_library().zeta_last_error().decode())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype | None = None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _v_dtype(v: torch.Tensor) -> int:
    if v.dtype == torch.float32:
        return ZETA_F32
    if v.dtype == torch.bfloat16:
        return ZETA_BF16
    raise ValueError(f"v must be float32 or bfloat16, got {v.dtype}")


def make_shape(B: int, H: int, N: int, dv: int, topk: int, v_dtype: int) -> ZetaShape:
    return ZetaShape(B, H, N, dv, topk, v_dtype, 0)


def zeta_workspace_bytes(shape: ZetaShape, kind: int) -> int:
    return int(load_library().zeta_workspace_bytes(ctypes.byref(shape), kind))


def zeta_workspace_bytes_ex(shape: ZetaShape, opts: ZetaSelectOpts | None, kind: int) -> int:
    return int(load_library().zeta_workspace_bytes_ex(ctypes.byref(shape), _opts_ref(opts), kind))


def workspace(shape: ZetaShape, kind: int, device,
              opts: ZetaSelectOpts | None = None) -> torch.Tensor:
    n = zeta_workspace_bytes_ex(shape, opts, kind)
    if n == 0:
        _check(ZETA_ERR_INVALID_ARGUMENT)
    return torch.empty(n, dtype=torch.uint8, device=device)


def zeta_tree_levels(N: int) -> int:
    return int(load_library().zeta_tree_levels(N))


def zeta_encode(x: torch.Tensor) -> torch.Tensor:
    """Z-order codes (int32 tensor holding the uint32 values) of points x [..., 3] fp32."""
    _dev(x, "x", torch.float32)
    if x.shape[-1] != 3:
        raise ValueError("x must have a trailing dimension of 3")
    codes = torch.empty(x.shape[:-1], dtype=torch.int32, device=x.device)
    _check(load_library().zeta_encode(_ptr(x), x.numel() // 3, _ptr(codes), _stream()))
    return codes


def zeta_build_tree(zk: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Merge-sort trees of key codes zk [BH, N] -> (asc, desc) int64 [BH, levels, N]."""
    _dev(zk, "zk", torch.int32)
    BH, N = zk.shape
    L = zeta_tree_levels(N)
    asc = torch.empty((BH, L, N), dtype=torch.int64, device=zk.device)
    desc = torch.empty_like(asc)
    _check(load_library().zeta_build_tree(BH, N, _ptr(zk), _ptr(asc), _ptr(desc), _stream()))
    return asc, desc


def _qk_shape(q: torch.Tensor, k: torch.Tensor):
    _dev(q, "q", torch.float32)
    _dev(k, "k", torch.float32)
    if q.dim() != 4 or q.shape[-1] != 3 or k.shape != q.shape:
        raise ValueError("q and k must both be [B, H, N, 3]")
    return q.shape[:3]


def zeta_select_ex(q: torch.Tensor, k: torch.Tensor, topk: int, opts: ZetaSelectOpts | None,
                   ws: torch.Tensor | None = None,
                   idx: torch.Tensor | None = None) -> torch.Tensor:
    """Selection (variant `opts`, None = exact causal): idx [B, H, N, topk] int32."""
    B, H, N = _qk_shape(q, k)
    shape = make_shape(B, H, N, 8, topk, ZETA_F32)
    if ws is None:
        ws = workspace(shape, ZETA_WS_SELECT, q.device, opts)
    if idx is None:
        idx = torch.empty((B, H, N, topk), dtype=torch.int32, device=q.device)
    _check(load_library().zeta_select_ex(ctypes.byref(shape), _opts_ref(opts), _ptr(q), _ptr(k),
                                         _ptr(idx), _ptr(ws), ws.numel(), _stream()))
    return idx


def zeta_select(q: torch.Tensor, k: torch.Tensor, topk: int,
                ws: torch.Tensor | None = None) -> torch.Tensor:
    """Exact causal top-k selection: idx [B, H, N, topk] int32, -1 padded."""
    B, H, N = _qk_shape(q, k)
    shape = make_shape(B, H, N, 8, topk, ZETA_F32)
    if ws is None:
        ws = workspace(shape, ZETA_WS_SELECT, q.device)
    idx = torch.empty((B, H, N, topk), dtype=torch.int32, device=q.device)
    _check(load_library().zeta_select(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(idx), _ptr(ws),
                                      ws.numel(), _stream()))
    return idx


def zeta_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, topk: int,
                opts: ZetaSelectOpts | None, ws: torch.Tensor | None = None,
                out: torch.Tensor | None = None,
                idx: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Forward with the selection variant `opts` (None = exact causal)."""
    B, H, N = _qk_shape(q, k)
    _dev(v, "v")
    _dev(gamma, "gamma", torch.float32)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, H, N) or gamma.shape != (H,):
        raise ValueError("v must be [B, H, N, dv] and gamma [H]")
    shape = make_shape(B, H, N, v.shape[3], topk, _v_dtype(v))
    if ws is None:
        ws = workspace(shape, ZETA_WS_FWD, q.device, opts)
    if out is None:
        out = torch.empty_like(v)
    if idx is None:
        idx = torch.empty((B, H, N, topk), dtype=torch.int32, device=q.device)
    _check(load_library().zeta_fwd_ex(ctypes.byref(shape), _opts_ref(opts), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(gamma), _ptr(out), _ptr(idx), _ptr(ws),
                                      ws.numel(), _stream()))
    return out, idx


def zeta_bwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                idx: torch.Tensor, dout: torch.Tensor, opts: ZetaSelectOpts | None,
                ws: torch.Tensor | None = None, grads: tuple | None = None):
    """Backward for a selection made with `opts` (only its causal flag matters)."""
    B, H, N = _qk_shape(q, k)
    _dev(v, "v")
    _dev(gamma, "gamma", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(dout, "dout", v.dtype)
    topk = idx.shape[-1]
    if tuple(idx.shape[:3]) != (B, H, N) or dout.shape != v.shape:
        raise ValueError("idx must be [B, H, N, topk] and dout shaped like v")
    shape = make_shape(B, H, N, v.shape[3], topk, _v_dtype(v))
    if ws is None:
        ws = workspace(shape, ZETA_WS_BWD, q.device, opts)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty((H,), dtype=torch.float32, device=q.device))
    dq, dk, dv, dg = grads
    _check(load_library().zeta_bwd_ex(ctypes.byref(shape), _opts_ref(opts), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(gamma), _ptr(idx), _ptr(dout), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ws), ws.numel(),
                                      _stream()))
    return dq, dk, dv, dg


def zeta_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, topk: int,
             ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
             idx: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Forward: (out [B,H,N,dv] in v's dtype, idx [B,H,N,topk] int32)."""
    B, H, N = _qk_shape(q, k)
    _dev(v, "v")
    _dev(gamma, "gamma", torch.float32)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, H, N) or gamma.shape != (H,):
        raise ValueError("v must be [B, H, N, dv] and gamma [H]")
    shape = make_shape(B, H, N, v.shape[3], topk, _v_dtype(v))
    if ws is None:
        ws = workspace(shape, ZETA_WS_FWD, q.device)
    if out is None:
        out = torch.empty_like(v)
    if idx is None:
        idx = torch.empty((B, H, N, topk), dtype=torch.int32, device=q.device)
    _check(load_library().zeta_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                   _ptr(out), _ptr(idx), _ptr(ws), ws.numel(), _stream()))
    return out, idx


def zeta_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
                     topk: int, out: torch.Tensor, idx: torch.Tensor):
    """Forward into caller-provided out / idx with the library's device scratch (no workspace,
    nothing allocated by the call)."""
    B, H, N = _qk_shape(q, k)
    _dev(v, "v")
    _dev(gamma, "gamma", torch.float32)
    _dev(out, "out", v.dtype)
    _dev(idx, "idx", torch.int32)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, H, N) or gamma.shape != (H,):
        raise ValueError("v must be [B, H, N, dv] and gamma [H]")
    if out.shape != v.shape or tuple(idx.shape) != (B, H, N, topk):
        raise ValueError("out must be shaped like v and idx [B, H, N, topk]")
    shape = make_shape(B, H, N, v.shape[3], topk, _v_dtype(v))
    _check(load_library().zeta_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(gamma), _ptr(out), _ptr(idx), _stream()))
    return out, idx


def zeta_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
             idx: torch.Tensor, dout: torch.Tensor, ws: torch.Tensor | None = None,
             grads: tuple | None = None):
    """Backward with the selection fixed: (dq fp32, dk fp32, dv v-dtype, dgamma fp32 [H])."""
    B, H, N = _qk_shape(q, k)
    _dev(v, "v")
    _dev(gamma, "gamma", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(dout, "dout", v.dtype)
    topk = idx.shape[-1]
    if tuple(idx.shape[:3]) != (B, H, N) or dout.shape != v.shape:
        raise ValueError("idx must be [B, H, N, topk] and dout shaped like v")
    shape = make_shape(B, H, N, v.shape[3], topk, _v_dtype(v))
    if ws is None:
        ws = workspace(shape, ZETA_WS_BWD, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty((H,), dtype=torch.float32, device=q.device))
    dq, dk, dv, dg = grads
    _check(load_library().zeta_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                   _ptr(idx), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                   _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv, dg


def zeta_probe_row_gather(table: torch.Tensor, row_bytes: int, groups: int, rows_per_group: int,
                          seed: int = 1, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement hook: scattered 16-lane row gathers from `table` (uint8 device tensor of
    table_rows * row_bytes bytes); returns the per-group sink words."""
    _dev(table, "table", torch.uint8)
    rows = table.numel() // row_bytes
    if sink is None:
        sink = torch.empty(groups, dtype=torch.int32, device=table.device)
    _check(load_library().zeta_probe_row_gather(_ptr(table), rows, row_bytes, groups,
                                                rows_per_group, seed, _ptr(sink), _stream()))
    return sink


class ZetaAttention(torch.autograd.Function):
    """Autograd wrapper: forward = zeta_fwd, backward = zeta_bwd (selection held fixed)."""

    @staticmethod
    def forward(ctx, q, k, v, gamma, topk: int):
        q, k, v, gamma = (t.contiguous() for t in (q, k, v, gamma))
        out, idx = zeta_fwd(q, k, v, gamma, topk)
        ctx.save_for_backward(q, k, v, gamma, idx)
        ctx.mark_non_differentiable(idx)
        return out, idx

    @staticmethod
    def backward(ctx, dout, _didx):
        q, k, v, gamma, idx = ctx.saved_tensors
        dq, dk, dv, dg = zeta_bwd(q, k, v, gamma, idx, dout.contiguous())
        return dq, dk, dv, dg, None


def zeta_attention(q, k, v, gamma, topk: int):
    """ZETA causal top-k attention with autograd: returns (out, idx)."""
    return ZetaAttention.apply(q, k, v, gamma, topk)
