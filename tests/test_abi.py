"""C-ABI checks that need no GPU: the library loads, exports every symbol include/zeta.h
declares, and every host-side validation path returns its documented status without
launching anything."""

import ctypes
import os
import re

import pytest
import torch

from order_retrieval_amd import zeta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zeta.h")

FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced by host validation


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(zeta.LIB_PATH):
        pytest.fail("libzeta.so is not built (run `python -m order_retrieval_amd.build`)")
    return zeta.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zeta_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert set(declared_functions()) == set(zeta.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_shares_torch_hip_runtime(lib):
    # torch is imported before the library, so the loader reuses torch's HIP runtime:
    # one runtime, one device context, and torch's streams are valid in the library.
    runtimes = zeta.hip_runtimes_mapped()
    assert len(runtimes) == 1 and "torch" in runtimes[0], runtimes


def shape(B=1, H=2, N=100, dv=64, topk=8, dt=zeta.ZETA_F32, reserved=0):
    s = zeta.make_shape(B, H, N, dv, topk, dt)
    s.reserved = reserved
    return s


def test_tree_levels(lib):
    assert [lib.zeta_tree_levels(n) for n in (0, 1, 2, 3, 4, 1000, 1024, 1025, 65536)] == \
        [0, 1, 2, 2, 3, 10, 11, 11, 17]


def test_status_strings(lib):
    for code, name in [(0, "ZETA_OK"), (1, "ZETA_ERR_INVALID_ARGUMENT"),
                       (2, "ZETA_ERR_UNSUPPORTED"), (3, "ZETA_ERR_WORKSPACE_TOO_SMALL"),
                       (4, "ZETA_ERR_HIP")]:
        assert lib.zeta_status_string(code).decode() == name


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(H=0), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(N=0), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(topk=0), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(topk=257), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(dv=12), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(dv=0), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(dv=520), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(dt=7), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(reserved=1), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(B=1024, H=1024, N=4096, topk=2), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(N=1 << 30), zeta.ZETA_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected_before_launch(lib, bad, code):
    s = shape(**bad)
    assert lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD) == 0
    st = lib.zeta_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code
    assert lib.zeta_last_error().decode() != ""
    st = lib.zeta_select(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code
    st = lib.zeta_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      FAKE, 1 << 40, None)
    assert st == code


def test_null_shape_and_pointers(lib):
    s = shape()
    ws = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
    assert ws > 0
    assert lib.zeta_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    for pos in range(7):
        args = [FAKE] * 7
        args[pos] = None
        st = lib.zeta_fwd(ctypes.byref(s), *args, ws, None)
        assert st == zeta.ZETA_ERR_INVALID_ARGUMENT, pos
    assert lib.zeta_select(ctypes.byref(s), None, FAKE, FAKE, FAKE, ws, None) == 1
    assert lib.zeta_encode(None, 10, FAKE, None) == 1
    assert lib.zeta_encode(FAKE, -1, FAKE, None) == 1
    assert lib.zeta_encode(None, 0, None, None) == 0  # empty input is a no-op
    assert lib.zeta_build_tree(0, 10, FAKE, FAKE, FAKE, None) == 1


def test_misaligned_pointers(lib):
    s = shape()
    ws = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
    odd = ctypes.c_void_p(0x100008)  # 8-byte but not 16-byte aligned
    assert lib.zeta_fwd(ctypes.byref(s), FAKE, FAKE, odd, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    assert lib.zeta_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, odd, ws, None) == 1
    q_odd = ctypes.c_void_p(0x100002)
    assert lib.zeta_select(ctypes.byref(s), q_odd, FAKE, FAKE, FAKE, ws, None) == 1


def test_workspace_too_small(lib):
    s = shape()
    for kind in (zeta.ZETA_WS_SELECT, zeta.ZETA_WS_FWD, zeta.ZETA_WS_BWD):
        assert lib.zeta_workspace_bytes(ctypes.byref(s), kind) > 0
    ws = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
    st = lib.zeta_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None)
    assert st == zeta.ZETA_ERR_WORKSPACE_TOO_SMALL
    wsb = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_BWD)
    st = lib.zeta_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      FAKE, wsb - 1, None)
    assert st == zeta.ZETA_ERR_WORKSPACE_TOO_SMALL


def test_noalloc_validates_before_any_launch(lib):
    # invalid shapes and NULL pointers as for zeta_fwd; a shape whose forward scratch exceeds
    # ZETA_NOALLOC_SCRATCH_BYTES is refused with the sizes in the message
    assert lib.zeta_fwd_noalloc(ctypes.byref(shape(topk=0)), *([FAKE] * 6), None) == 1
    assert lib.zeta_fwd_noalloc(ctypes.byref(shape()), None, *([FAKE] * 5), None) == 1
    big = shape(B=1, H=16, N=65536, dv=128, topk=32, dt=zeta.ZETA_BF16)
    assert lib.zeta_workspace_bytes(ctypes.byref(big), zeta.ZETA_WS_FWD) > 128 << 20
    st = lib.zeta_fwd_noalloc(ctypes.byref(big), *([FAKE] * 6), None)
    assert st == zeta.ZETA_ERR_WORKSPACE_TOO_SMALL
    assert "ZETA_NOALLOC_SCRATCH_BYTES" in lib.zeta_last_error().decode()
    fits = shape(B=1, H=8, N=65536, dv=128, topk=32, dt=zeta.ZETA_BF16)
    assert lib.zeta_workspace_bytes(ctypes.byref(fits), zeta.ZETA_WS_FWD) <= 128 << 20


@pytest.mark.parametrize("args", [
    (None, 1024, 256, 100, 32), (FAKE, 1000, 256, 100, 32), (FAKE, 1024, 8, 100, 32),
    (FAKE, 1024, 272, 100, 32), (FAKE, 1024, 256, 0, 32), (FAKE, 1024, 256, 100, 12),
    (ctypes.c_void_p(0x100008), 1024, 256, 100, 32),
])
def test_probe_validates_before_launch(lib, args):
    table, rows, rb, groups, per = args
    assert lib.zeta_probe_row_gather(table, rows, rb, groups, per, 1, FAKE, None) == 1


def test_workspace_grows_with_shape(lib):
    a = lib.zeta_workspace_bytes(ctypes.byref(shape(N=1000)), zeta.ZETA_WS_FWD)
    b = lib.zeta_workspace_bytes(ctypes.byref(shape(N=4000)), zeta.ZETA_WS_FWD)
    assert 0 < a < b
    assert lib.zeta_workspace_bytes(ctypes.byref(shape()), 9) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_hip_error(lib):
    s = shape()
    ws = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
    st = lib.zeta_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert st == zeta.ZETA_ERR_HIP
    assert "device" in lib.zeta_last_error().decode()
    assert lib.zeta_encode(FAKE, 10, FAKE, None) == zeta.ZETA_ERR_HIP


# --------------------------------------------------------------------------- variant options
def opts(**kw):
    base = dict(mode=zeta.ZETA_SELECT_EXACT, causal=1, bits=10, chunks=0, curves=0, reserved=0)
    base.update(kw)
    return zeta.ZetaSelectOpts(base["mode"], base["causal"], base["bits"], base["chunks"],
                               base["curves"], base["reserved"])


@pytest.mark.parametrize("bad,code", [
    (dict(mode=3), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(bits=11), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(reserved=1), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(mode=zeta.ZETA_SELECT_CHUNKED, chunks=0), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(mode=zeta.ZETA_SELECT_CHUNKED, chunks=2000), zeta.ZETA_ERR_INVALID_ARGUMENT),
    (dict(mode=zeta.ZETA_SELECT_CHUNKED, chunks=8, causal=0), zeta.ZETA_ERR_UNSUPPORTED),
    (dict(mode=zeta.ZETA_SELECT_CURVES, curves=4), zeta.ZETA_ERR_INVALID_ARGUMENT),
])
def test_invalid_options_rejected_before_launch(lib, bad, code):
    s = shape()
    o = opts(**bad)
    assert lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(o), zeta.ZETA_WS_FWD) == 0
    st = lib.zeta_select_ex(ctypes.byref(s), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code, lib.zeta_last_error()
    st = lib.zeta_fwd_ex(ctypes.byref(s), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         1 << 40, None)
    assert st == code
    st = lib.zeta_bwd_ex(ctypes.byref(s), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code


def test_curves_need_topk_of_at_least_the_curve_count(lib):
    s = shape(topk=2)
    o = opts(mode=zeta.ZETA_SELECT_CURVES, curves=3)
    assert lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(o), zeta.ZETA_WS_FWD) == 0


def test_null_options_equal_the_plain_calls(lib):
    s = shape()
    for kind in (zeta.ZETA_WS_SELECT, zeta.ZETA_WS_FWD, zeta.ZETA_WS_BWD):
        assert (lib.zeta_workspace_bytes_ex(ctypes.byref(s), None, kind) ==
                lib.zeta_workspace_bytes(ctypes.byref(s), kind) > 0)
    # default options describe the same selection as NULL
    o = opts()
    assert (lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(o), zeta.ZETA_WS_FWD) ==
            lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD))


def test_causal_tree_skips_the_top_level(lib):
    # under the causal mask the level of N keys is read only by the last query when N is a
    # power of two, which takes it as two runs of the level below: one level fewer per tree
    for N, fewer in ((65536, 1), (4096, 1), (1000, 0), (64, 0), (128, 1)):
        s = shape(B=2, H=2, N=N, topk=32)
        nc = opts(causal=0)
        causal = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
        full = lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(nc), zeta.ZETA_WS_FWD)
        assert full - causal == fewer * 2 * 8 * 2 * 2 * N, N


def test_variant_workspaces(lib):
    s = shape(N=1000, topk=32)
    base = lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_FWD)
    curves = opts(mode=zeta.ZETA_SELECT_CURVES, curves=3)
    assert lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(curves), zeta.ZETA_WS_FWD) > base
    # one chunk of 1024 positions reads a single tree level (above the top one of N = 1000),
    # the only one it stores; the exact search stores levels 6 .. 9 (runs of 2K = 64 and up)
    one = opts(mode=zeta.ZETA_SELECT_CHUNKED, chunks=1)
    w1 = lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(one), zeta.ZETA_WS_FWD)
    assert 0 < w1 < base
    assert base - w1 >= 2 * 8 * 2 * 1000  # two trees, at least two levels fewer
    nc = opts(causal=0)
    assert (lib.zeta_workspace_bytes_ex(ctypes.byref(s), ctypes.byref(nc), zeta.ZETA_WS_BWD) >
            lib.zeta_workspace_bytes(ctypes.byref(s), zeta.ZETA_WS_BWD))
