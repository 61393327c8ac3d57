"""GPU parity of the selection variants (through the C ABI's _ex calls) against the oracle:
the unmasked exact selection, the chunked causal search and several curves, and the
forward and backward passes on the selections they return (slots holding -1 anywhere,
queries with no selected key).

Selections are compared bit for bit; outputs and gradients within the tolerance rule of
gpu_common.
"""

import numpy as np
import pytest
import torch

import oracle
from order_retrieval_amd import inputs
from order_retrieval_amd import zeta as Z
from gpu_common import assert_close, device_inputs, log, sample_rows, to_dev, to_np

pytestmark = pytest.mark.gpu

CFG = inputs.CONFIGS


def W(name, B, H, N, dv, topk, vt=inputs.F32, dist="normal", seed=0, backward=False):
    return inputs.Workload(name, B, H, N, dv, topk, vt, dist, None, seed, backward)


def opts_of(kind):
    """kind: ('exact', causal) | ('chunked', C) | ('curves', P, causal)."""
    if kind[0] == "exact":
        return Z.select_opts(Z.ZETA_SELECT_EXACT, causal=kind[1])
    if kind[0] == "chunked":
        return Z.select_opts(Z.ZETA_SELECT_CHUNKED, causal=True, chunks=kind[1])
    return Z.select_opts(Z.ZETA_SELECT_CURVES, causal=kind[2], curves=kind[1])


def causal_of(kind):
    return kind[1] if kind[0] == "exact" else (True if kind[0] == "chunked" else kind[2])


def oracle_select(kind, x, topk, rows=None):
    q, k = x["q"], x["k"]
    N = q.shape[2]
    if kind[0] == "exact":
        return oracle.select_ex(q, k, topk, 10, causal=kind[1], rows=rows)
    if kind[0] == "chunked":
        return oracle.select_chunked(oracle.encode(q), oracle.encode(k), N, topk, kind[1],
                                     rows=rows)
    return oracle.select_multi(q, k, topk, kind[1], causal=kind[2], rows=rows)


KINDS = [("exact", False), ("chunked", 1), ("chunked", 4), ("chunked", 32), ("curves", 3, True),
         ("curves", 6, True), ("curves", 3, False)]


def _name(kind):
    return "-".join(str(t) for t in kind)


# ----------------------------------------------------------------------------- selection
def _assert_rejected(w, opts):
    """topk below the curve count: the call is refused before any launch, idx untouched."""
    x = inputs.make_inputs(w)
    idx = torch.full((w.B, w.H, w.N, w.topk), 7, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    with pytest.raises(Z.ZetaError) as e:
        Z.zeta_select_ex(to_dev(x["q"]), to_dev(x["k"]), w.topk, opts, ws=ws, idx=idx)
    assert e.value.status == Z.ZETA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.all(idx == 7)


def _select_check(w, kind, rows=None):
    x = inputs.make_inputs(w)
    idx = Z.zeta_select_ex(to_dev(x["q"]), to_dev(x["k"]), w.topk, opts_of(kind))
    torch.cuda.synchronize()
    got = to_np(idx).reshape(-1, w.topk)
    ref = oracle_select(kind, x, w.topk, rows)
    np.testing.assert_array_equal(got if rows is None else got[rows], ref)
    return got


@pytest.mark.parametrize("kind", KINDS, ids=_name)
@pytest.mark.parametrize("name", ["tiny", "multihead"])
def test_variant_select_bit_exact_full(name, kind):
    log(f"variant select {name} {kind}")
    _select_check(CFG[name], kind)


@pytest.mark.parametrize("kind", [("exact", False), ("chunked", 32), ("curves", 3, True)],
                         ids=_name)
def test_variant_select_sampled_long(kind):
    w = CFG["long_fwd"]
    rows = sample_rows(w, 300 if kind[0] != "curves" else 600, seed=9)
    log(f"variant select long {kind}: {rows.size} rows")
    _select_check(w, kind, rows)


@pytest.mark.parametrize("B,H,N,topk,dist", [
    (1, 1, 1, 1, "normal"), (2, 1, 3, 4, "discrete"), (1, 2, 777, 5, "clustered"),
    (1, 1, 1000, 32, "normal"), (2, 2, 1025, 64, "discrete"), (1, 1, 2049, 16, "constant"),
    (1, 3, 300, 48, "clustered"), (1, 1, 70, 7, "normal"),
])
@pytest.mark.parametrize("kind", KINDS + [("chunked", 1024), ("chunked", 3), ("curves", 6, False)],
                         ids=_name)
def test_variant_select_edge_shapes(B, H, N, topk, dist, kind):
    log(f"variant select edge B={B} H={H} N={N} k={topk} {dist} {kind}")
    if kind[0] == "curves" and topk < kind[1]:
        _assert_rejected(W("ve", B, H, N, 8, topk, dist=dist, seed=N + topk), opts_of(kind))
        return
    _select_check(W("ve", B, H, N, 8, topk, dist=dist, seed=N + topk), kind)


# ----------------------------------------------------------------------------- forward
def _forward_check(w, kind, rows=None):
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    out, idx = Z.zeta_fwd_ex(d["q"], d["k"], d["v"], d["gamma"], w.topk, opts_of(kind))
    torch.cuda.synchronize()
    got_idx = to_np(idx).reshape(-1, w.topk)
    ref_idx = oracle_select(kind, x, w.topk, rows)
    np.testing.assert_array_equal(got_idx if rows is None else got_idx[rows], ref_idx)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gamma"], ref_idx, w.v_dtype == inputs.BF16,
                         rows=rows)
    got = to_np(out).reshape(-1, w.dv)
    assert_close(got if rows is None else got[rows], ref, w.v_dtype, f"o {w.name} {kind}",
                 bf16_output=w.v_dtype == inputs.BF16)
    return ref_idx


@pytest.mark.parametrize("kind", KINDS, ids=_name)
@pytest.mark.parametrize("name", ["tiny", "multihead"])
def test_variant_forward_full(name, kind):
    log(f"variant forward {name} {kind}")
    w = CFG[name]
    ref_idx = _forward_check(w, kind)
    if kind[0] == "chunked" and oracle.chunk_len(w.N, kind[1]) > w.topk:
        # windows narrower than a chunk: some early queries see no key j <= i
        assert (ref_idx < 0).all(axis=1).any(), "expected queries with an empty selection"


@pytest.mark.parametrize("kind", [("exact", False), ("chunked", 8), ("curves", 3, True)],
                         ids=_name)
@pytest.mark.parametrize("N,dv,vt", [(1000, 136, inputs.BF16), (333, 512, inputs.F32),
                                     (64, 24, inputs.F32)])
def test_variant_forward_edge_shapes(N, dv, vt, kind):
    log(f"variant forward edge N={N} dv={dv} {vt} {kind}")
    _forward_check(W("vf", 2, 2, N, dv, 16, vt, "clustered", seed=N + dv), kind)


@pytest.mark.parametrize("kind", [("chunked", 4), ("chunked", 16), ("curves", 3, True),
                                  ("curves", 6, False), ("exact", False)], ids=_name)
@pytest.mark.parametrize("B,H,N,topk,dist", [(1, 2, 3000, 128, "clustered"),
                                             (2, 1, 1500, 256, "normal"),
                                             (1, 1, 700, 96, "discrete")])
def test_variant_wide_topk(B, H, N, topk, dist, kind):
    log(f"variant wide k={topk} B={B} H={H} N={N} {dist} {kind}")
    w = W("vw", B, H, N, 32, topk, inputs.BF16, dist, seed=N + topk, backward=True)
    _backward_check(w, kind)


def test_variant_forward_sampled_long():
    w = CFG["long_fwd"]
    rows = sample_rows(w, 300, seed=10)
    for kind in [("exact", False), ("chunked", 32)]:
        log(f"variant forward long {kind}: {rows.size} rows")
        _forward_check(w, kind, rows)


# ----------------------------------------------------------------------------- backward
def _backward_check(w, kind):
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    bf = w.v_dtype == inputs.BF16
    o = opts_of(kind)
    _, idx = Z.zeta_fwd_ex(d["q"], d["k"], d["v"], d["gamma"], w.topk, o)
    dq, dk, dv, dg = Z.zeta_bwd_ex(d["q"], d["k"], d["v"], d["gamma"], idx, d["dout"], o)
    torch.cuda.synchronize()
    ref_idx = oracle_select(kind, x, w.topk)
    np.testing.assert_array_equal(to_np(idx).reshape(-1, w.topk), ref_idx)
    rq, rk, rv, rg = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], ref_idx, bf)
    assert_close(to_np(dq).reshape(-1, 3), rq, w.v_dtype, f"dq {kind}")
    assert_close(to_np(dk), rk, w.v_dtype, f"dk {kind}")
    assert_close(to_np(dv), rv, w.v_dtype, f"dv {kind}", bf16_output=bf)
    assert_close(to_np(dg), rg, w.v_dtype, f"dgamma {kind}")


@pytest.mark.parametrize("kind", KINDS, ids=_name)
@pytest.mark.parametrize("name", ["tiny", "multihead"])
def test_variant_backward_full(name, kind):
    log(f"variant backward {name} {kind}")
    _backward_check(inputs.Workload(**{**CFG[name].__dict__, "backward": True}), kind)


@pytest.mark.parametrize("kind", [("exact", False), ("chunked", 4), ("curves", 6, True)],
                         ids=_name)
@pytest.mark.parametrize("B,H,N,dv,topk,vt", [(1, 1, 1, 8, 6, inputs.F32),
                                              (2, 1, 700, 64, 32, inputs.BF16),
                                              (1, 2, 300, 512, 12, inputs.F32),
                                              (1, 1, 70000, 8, 8, inputs.BF16)])
def test_variant_backward_edge_shapes(B, H, N, dv, topk, vt, kind):
    log(f"variant backward edge B={B} H={H} N={N} dv={dv} k={topk} {vt} {kind}")
    w = W("vb", B, H, N, dv, topk, vt, "clustered", seed=N + topk, backward=True)
    if N > 10000:
        _backward_sampled(w, kind)
    else:
        _backward_check(w, kind)


def _backward_sampled(w, kind):
    """Large N: dq of sampled queries, and dk / dv of the keys that only the last 128 queries
    can select under the causal mask (non-causal: keys of a small all-query brute force are
    out of reach, so only dq there)."""
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    bf = w.v_dtype == inputs.BF16
    o = opts_of(kind)
    _, idx = Z.zeta_fwd_ex(d["q"], d["k"], d["v"], d["gamma"], w.topk, o)
    dq, dk, dv, dg = Z.zeta_bwd_ex(d["q"], d["k"], d["v"], d["gamma"], idx, d["dout"], o)
    torch.cuda.synchronize()
    N = w.N
    rows = sample_rows(w, 200, seed=11)
    ref_idx = oracle_select(kind, x, w.topk, rows)
    np.testing.assert_array_equal(to_np(idx).reshape(-1, w.topk)[rows], ref_idx)
    rq, _, _, _ = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], ref_idx, bf,
                                  rows=rows)
    assert_close(to_np(dq).reshape(-1, 3)[rows], rq, w.v_dtype, f"dq sampled {kind}")
    if causal_of(kind):
        BH = w.B * w.H
        tail = np.concatenate([np.arange(bh * N + N - 128, bh * N + N) for bh in range(BH)])
        tidx = oracle_select(kind, x, w.topk, tail)
        _, rk, rv, _ = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], tidx, bf,
                                       rows=tail)
        gk = to_np(dk).reshape(BH, N, 3)[:, N - 128:]
        gv = to_np(dv).reshape(BH, N, -1)[:, N - 128:]
        assert_close(gk, rk.reshape(BH, N, 3)[:, N - 128:], w.v_dtype, f"dk tail {kind}")
        assert_close(gv, rv.reshape(BH, N, -1)[:, N - 128:], w.v_dtype, f"dv tail {kind}",
                     bf16_output=bf)


def test_backward_of_selection_with_holes_and_empty_rows():
    """zeta_bwd on an index tensor with -1 in arbitrary slots and whole empty rows (what the
    approximate selections can return), causal and not."""
    w = W("holes", 2, 2, 500, 40, 12, inputs.F32, "normal", seed=21, backward=True)
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    rng = np.random.default_rng(3)
    for causal in (True, False):
        idx = oracle.select_ex(x["q"], x["k"], w.topk, 10, causal=causal)
        idx[rng.random(idx.shape) < 0.3] = -1
        idx[rng.integers(0, idx.shape[0], 40)] = -1
        o = Z.select_opts(Z.ZETA_SELECT_EXACT, causal=causal)
        gidx = to_dev(idx.reshape(w.B, w.H, w.N, w.topk))
        dq, dk, dv, dg = Z.zeta_bwd_ex(d["q"], d["k"], d["v"], d["gamma"], gidx, d["dout"], o)
        torch.cuda.synchronize()
        rq, rk, rv, rg = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], idx,
                                         False)
        assert_close(to_np(dq).reshape(-1, 3), rq, w.v_dtype, f"dq holes causal={causal}")
        assert_close(to_np(dk), rk, w.v_dtype, f"dk holes causal={causal}")
        assert_close(to_np(dv), rv, w.v_dtype, f"dv holes causal={causal}")
        assert_close(to_np(dg), rg, w.v_dtype, f"dgamma holes causal={causal}")


def test_backward_of_all_empty_selection_is_zero():
    w = W("empty", 1, 2, 300, 16, 8, inputs.BF16, "normal", seed=22, backward=True)
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    idx = torch.full((w.B, w.H, w.N, w.topk), -1, dtype=torch.int32, device="cuda")
    dq, dk, dv, dg = Z.zeta_bwd(d["q"], d["k"], d["v"], d["gamma"], idx, d["dout"])
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dg):
        assert torch.count_nonzero(t.float()).item() == 0


def test_variant_deterministic():
    w = inputs.Workload(**{**CFG["multihead"].__dict__, "backward": True})
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    o = opts_of(("chunked", 8))
    res = []
    for _ in range(2):
        out, idx = Z.zeta_fwd_ex(d["q"], d["k"], d["v"], d["gamma"], w.topk, o)
        g = Z.zeta_bwd_ex(d["q"], d["k"], d["v"], d["gamma"], idx, d["dout"], o)
        torch.cuda.synchronize()
        res.append([to_np(t).copy() for t in (out, idx) + tuple(g)])
    for a, b in zip(*res):
        np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------- 12-bit cells
KINDS12 = [("exact", True), ("exact", False), ("chunked", 4), ("curves", 3, True)]


def opts12(kind):
    o = opts_of(kind)
    o.bits = 12
    return o


def oracle_select12(kind, x, topk, rows=None):
    q, k = x["q"], x["k"]
    N = q.shape[2]
    if kind[0] == "exact":
        return oracle.select_ex(q, k, topk, 12, causal=kind[1], rows=rows)
    if kind[0] == "chunked":
        return oracle.select_chunked(oracle.encode_ex(q, 12), oracle.encode_ex(k, 12), N, topk,
                                     kind[1], rows=rows)
    return oracle.select_multi(q, k, topk, kind[1], causal=kind[2], rows=rows, bits=12)


def _select12_check(w, kind, rows=None):
    x = inputs.make_inputs(w)
    idx = Z.zeta_select_ex(to_dev(x["q"]), to_dev(x["k"]), w.topk, opts12(kind))
    torch.cuda.synchronize()
    got = to_np(idx).reshape(-1, w.topk)
    np.testing.assert_array_equal(got if rows is None else got[rows],
                                  oracle_select12(kind, x, w.topk, rows))


@pytest.mark.parametrize("kind", KINDS12, ids=_name)
@pytest.mark.parametrize("name", ["tiny", "multihead", "clustered_small"])
def test_12bit_select_bit_exact(name, kind):
    w = CFG[name] if name != "clustered_small" else W("c12", 2, 2, 3000, 8, 64, dist="clustered",
                                                     seed=31)
    log(f"12-bit select {name} {kind}")
    _select12_check(w, kind)


@pytest.mark.parametrize("B,H,N,topk,dist", [
    (1, 1, 1, 1, "normal"), (2, 1, 3, 4, "discrete"), (1, 2, 777, 5, "clustered"),
    (2, 2, 1025, 64, "discrete"), (1, 1, 2049, 16, "constant"),
])
@pytest.mark.parametrize("kind", KINDS12, ids=_name)
def test_12bit_select_edge_shapes(B, H, N, topk, dist, kind):
    log(f"12-bit select edge B={B} H={H} N={N} k={topk} {dist} {kind}")
    if kind[0] == "curves" and topk < kind[1]:
        _assert_rejected(W("v12", B, H, N, 8, topk, dist=dist, seed=N + topk), opts12(kind))
        return
    _select12_check(W("v12", B, H, N, 8, topk, dist=dist, seed=N + topk), kind)


def test_12bit_select_sampled_long():
    w = CFG["long_fwd"]
    rows = sample_rows(w, 400, seed=12)
    log(f"12-bit select long: {rows.size} rows")
    _select12_check(w, ("exact", True), rows)


@pytest.mark.parametrize("kind", [("exact", True), ("chunked", 4)], ids=_name)
def test_12bit_forward_backward_full(kind):
    w = inputs.Workload(**{**CFG["tiny"].__dict__, "backward": True})
    x = inputs.make_inputs(w)
    d = device_inputs(w, x)
    o = opts12(kind)
    out, idx = Z.zeta_fwd_ex(d["q"], d["k"], d["v"], d["gamma"], w.topk, o)
    dq, dk, dv, dg = Z.zeta_bwd_ex(d["q"], d["k"], d["v"], d["gamma"], idx, d["dout"], o)
    torch.cuda.synchronize()
    ref_idx = oracle_select12(kind, x, w.topk)
    np.testing.assert_array_equal(to_np(idx).reshape(-1, w.topk), ref_idx)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gamma"], ref_idx, False)
    assert_close(to_np(out).reshape(-1, w.dv), ref, w.v_dtype, f"o 12-bit {kind}")
    rq, rk, rv, rg = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], ref_idx, False)
    assert_close(to_np(dq).reshape(-1, 3), rq, w.v_dtype, f"dq 12-bit {kind}")
    assert_close(to_np(dk), rk, w.v_dtype, f"dk 12-bit {kind}")
    assert_close(to_np(dv), rv, w.v_dtype, f"dv 12-bit {kind}")
    assert_close(to_np(dg), rg, w.v_dtype, f"dgamma 12-bit {kind}")


def test_12bit_differs_from_10bit_where_cells_split():
    """The finer grid separates points that share a 10-bit cell, so the two selections
    differ on clustered data (and each matches its own oracle above)."""
    w = W("split", 1, 1, 2000, 8, 16, dist="clustered", seed=33)
    x = inputs.make_inputs(w)
    a = to_np(Z.zeta_select_ex(to_dev(x["q"]), to_dev(x["k"]), w.topk, opts_of(("exact", True))))
    b = to_np(Z.zeta_select_ex(to_dev(x["q"]), to_dev(x["k"]), w.topk, opts12(("exact", True))))
    assert (a != b).any()
