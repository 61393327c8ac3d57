"""zeta_fwd_noalloc (the forward with the library's device scratch, no workspace argument)
against zeta_fwd through the C ABI: two calls in a row, the second with a smaller input, each
compared with zeta_fwd on the same inputs (indices bit for bit, outputs bit for bit: the same
kernels run on the same data)."""

import ctypes

import numpy as np
import pytest
import torch

from order_retrieval_amd import inputs
from order_retrieval_amd import zeta as Z
from gpu_common import device_inputs, log

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, d, topk, out, idx):
    B, H, N, _ = d["q"].shape
    shape = Z.make_shape(B, H, N, d["v"].shape[3], topk,
                         Z.ZETA_BF16 if d["v"].dtype == torch.bfloat16 else Z.ZETA_F32)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.zeta_fwd_noalloc(ctypes.byref(shape), ctypes.c_void_p(d["q"].data_ptr()),
                                ctypes.c_void_p(d["k"].data_ptr()),
                                ctypes.c_void_p(d["v"].data_ptr()),
                                ctypes.c_void_p(d["gamma"].data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                stream)


def test_noalloc_forward_matches_zeta_fwd_twice_second_smaller():
    lib = Z.load_library()
    cases = [inputs.CONFIGS["long_fwd"],  # B1 H8 N65536 dV128 k32 bf16: about 101 MB of scratch
             inputs.Workload("small", 1, 2, 3000, 24, 16, inputs.F32, "clustered", None, seed=5)]
    for w in cases:
        log(f"noalloc forward {w.name}: B{w.B} H{w.H} N{w.N} dV{w.dv} k{w.topk} {w.v_dtype}")
        x = inputs.make_inputs(w)
        d = device_inputs(w, x)
        ref_out, ref_idx = Z.zeta_fwd(d["q"], d["k"], d["v"], d["gamma"], w.topk)
        out = torch.full_like(ref_out, float("nan"))
        idx = torch.full_like(ref_idx, -7)
        st = _call_noalloc(lib, d, w.topk, out, idx)
        assert st == Z.ZETA_OK, lib.zeta_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        np.testing.assert_array_equal(out.view(torch.int16 if out.dtype == torch.bfloat16
                                               else torch.int32).cpu().numpy(),
                                      ref_out.view(torch.int16 if out.dtype == torch.bfloat16
                                                   else torch.int32).cpu().numpy())


def test_noalloc_rejects_oversized_shape_outputs_untouched():
    lib = Z.load_library()
    w = inputs.Workload("big", 1, 16, 65536, 8, 32, inputs.F32, "normal", None, seed=6)
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    out = torch.full_like(d["v"], 3.0)
    idx = torch.full((w.B, w.H, w.N, w.topk), 5, dtype=torch.int32, device="cuda")
    st = _call_noalloc(lib, d, w.topk, out, idx)
    assert st == Z.ZETA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(idx == 5)
