"""Pins of the oracle's selection variants (CPU only): the pages' 12-bit precision, the
unmasked case, the chunked causal search, several curves, and the Euclidean top-k used by
the recall diagnostic.

Each test checks the oracle against something other than itself: hand-worked tables
(tests/golden), exact relations between the 10- and 12-bit forms, reductions of a variant
to the exact selection, brute force in numpy, and the empty-selection rule.
"""

import os

import numpy as np
import pytest

import oracle
from order_retrieval_amd import inputs


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _opt(tok, name, default=None):
    for t in tok:
        if t.startswith(name + "="):
            return int(t.split("=")[1])
    return default


# --------------------------------------------------------------------------- 12-bit codes
def test_quantiser12_hand_table(golden_dir):
    for x, cell in _read_table(os.path.join(golden_dir, "quantiser12_cells.txt")):
        xf = float(np.float32(float(x)))
        assert oracle.cell12(xf) == int(cell), (x, oracle.cell12(xf), cell)


def test_interleave36_hand_table(golden_dir):
    for c0, c1, c2, z in _read_table(os.path.join(golden_dir, "morton36.txt")):
        assert oracle.interleave36(int(c0), int(c1), int(c2)) == int(z), (c0, c1, c2, z)


def test_cell12_refines_cell10():
    """Both grids cover [-4, 4); 4 fine cells make one coarse cell, so cell12 >> 2 == cell."""
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.normal(0, 2, 4000), rng.uniform(-4.01, 4.01, 4000),
                         np.arange(-1030, 1030) / 256.0, [-4.0, 4.0, -1e-9, 1e-9, -0.0]])
    for x in xs.astype(np.float32):
        assert oracle.cell12(float(x)) >> 2 == oracle.cell(float(x)), x


def test_code36_refines_code30():
    """Dropping the two low bits of every cell drops the six low bits of the code."""
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1.5, (3000, 3)).astype(np.float32)
    z36 = oracle.encode_ex(x, 12)
    z30 = oracle.encode(x)
    np.testing.assert_array_equal(z36 >> np.uint64(6), z30.astype(np.uint64))


def test_encode_permutation_moves_coordinates():
    """Axis a of a permuted curve reads coordinate perm[a]: same as permuting the columns."""
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, (500, 3)).astype(np.float32)
    for perm in [(1, 2, 0), (2, 0, 1), (0, 2, 1), (2, 1, 0)]:
        for bits in (10, 12):
            np.testing.assert_array_equal(oracle.encode_ex(x, bits, perm),
                                          oracle.encode_ex(np.ascontiguousarray(x[:, perm]), bits))


# --------------------------------------------------------------------------- hand cases
def _variant_cases(path):
    cases, cur = [], None
    for tok in _read_table(path):
        if tok[0] == "case":
            cur = {"name": tok[1], "mode": tok[2], "k": _opt(tok, "k"), "C": _opt(tok, "C"),
                   "rows": []}
            cases.append(cur)
        elif tok[0] in ("zk", "zq"):
            cur[tok[0]] = np.array([int(t) for t in tok[1:]], dtype=np.uint64)
        else:
            cur["rows"].append([int(t) for t in tok])
    return cases


def test_variant_hand_examples(golden_dir):
    for case in _variant_cases(os.path.join(golden_dir, "select_variants_hand.txt")):
        N, K = case["zk"].size, case["k"]
        if case["mode"] == "noncausal":
            idx = oracle.select_codes64(case["zq"], case["zk"], N, K, causal=False)
        elif case["mode"] == "causal":
            idx = oracle.select_codes64(case["zq"], case["zk"], N, K, causal=True)
        else:
            idx = oracle.select_chunked(case["zq"].astype(np.uint32), case["zk"].astype(np.uint32),
                                        N, K, case["C"])
        np.testing.assert_array_equal(idx, np.array(case["rows"]), err_msg=case["name"])


def test_multi_curve_hand_examples(golden_dir):
    cases, cur = [], None
    for tok in _read_table(os.path.join(golden_dir, "select_multi_hand.txt")):
        if tok[0] == "case":
            cur = {"name": tok[1], "P": _opt(tok, "P"), "k": _opt(tok, "k"), "kp": [], "qp": [],
                   "rows": []}
            cases.append(cur)
        elif tok[0] == "k":
            cur["kp"].append([float(t) for t in tok[1:]])
        elif tok[0] == "q":
            cur["qp"].append([float(t) for t in tok[1:]])
        else:
            cur["rows"].append([int(t) for t in tok])
    for c in cases:
        q = np.array(c["qp"], dtype=np.float32)[None, None]
        k = np.array(c["kp"], dtype=np.float32)[None, None]
        idx = oracle.select_multi(q, k, c["k"], c["P"])
        np.testing.assert_array_equal(idx, np.array(c["rows"]), err_msg=c["name"])
        # 12-bit cells: coordinates 0 and 1/512 are cells 2048 and 2049, whose codes differ
        # by the same low offsets, so the same selection follows
        idx12 = oracle.select_multi(q / 4, k / 4, c["k"], c["P"], bits=12)
        np.testing.assert_array_equal(idx12, np.array(c["rows"]), err_msg=c["name"] + " 12-bit")


# --------------------------------------------------------------------------- exact, 64-bit
def _brute(zq, zk, N, K, causal):
    """numpy brute force of the exact selection (lexsort of (|dz|, j))."""
    BH = zq.size // N
    zq = zq.reshape(BH, N).astype(object)
    zk = zk.reshape(BH, N).astype(object)
    out = np.full((BH * N, K), -1, dtype=np.int64)
    for bh in range(BH):
        for i in range(N):
            n = i + 1 if causal else N
            d = np.array([abs(int(zq[bh, i]) - int(zk[bh, j])) for j in range(n)], dtype=object)
            order = sorted(range(n), key=lambda j: (d[j], j))[:K]
            out[bh * N + i, :len(order)] = order
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dist", ["normal", "clustered", "discrete"])
def test_select64_matches_brute_force(causal, dist):
    w = inputs.Workload("t", 1, 2, 40, 8, 6, dist=dist, seed=11)
    x = inputs.make_inputs(w)
    for bits in (10, 12):
        zq, zk = oracle.encode_ex(x["q"], bits), oracle.encode_ex(x["k"], bits)
        idx = oracle.select_codes64(zq, zk, w.N, w.topk, causal)
        np.testing.assert_array_equal(idx, _brute(zq.reshape(-1), zk.reshape(-1), w.N, w.topk,
                                                  causal))


def test_select64_on_30_bit_codes_matches_exact_select():
    w = inputs.Workload("t", 1, 2, 300, 8, 16, dist="clustered", seed=12)
    x = inputs.make_inputs(w)
    zq, zk = oracle.encode(x["q"]), oracle.encode(x["k"])
    a = oracle.select_codes(zq, zk, w.N, w.topk)
    b = oracle.select_codes64(zq.astype(np.uint64), zk.astype(np.uint64), w.N, w.topk)
    np.testing.assert_array_equal(a, b)
    # scaling every code by 2^6 keeps every |dz| order
    c = oracle.select_codes64(zq.astype(np.uint64) << np.uint64(6),
                              zk.astype(np.uint64) << np.uint64(6), w.N, w.topk)
    np.testing.assert_array_equal(a, c)


def test_noncausal_last_query_equals_causal():
    w = inputs.Workload("t", 1, 2, 200, 8, 12, dist="normal", seed=13)
    x = inputs.make_inputs(w)
    nc = oracle.select_ex(x["q"], x["k"], w.topk, 10, causal=False).reshape(2, w.N, -1)
    ca = oracle.select_ex(x["q"], x["k"], w.topk, 10, causal=True).reshape(2, w.N, -1)
    np.testing.assert_array_equal(nc[:, -1], ca[:, -1])
    assert np.all(nc >= 0)  # k <= N: every slot filled


def test_noncausal_all_equal_codes_takes_first_positions():
    N, K = 50, 7
    z = np.full(N, 12345, dtype=np.uint64)
    idx = oracle.select_codes64(z, z, N, K, causal=False)
    np.testing.assert_array_equal(idx, np.tile(np.arange(K), (N, 1)))


# --------------------------------------------------------------------------- chunked
def test_chunk_len():
    assert oracle.chunk_len(65536, 32) == 2048
    assert oracle.chunk_len(65536, 4) == 16384
    assert oracle.chunk_len(1000, 8) == 128   # ceil(1000/8) = 125 -> 128, 8 chunks
    assert oracle.chunk_len(1025, 8) == 256   # 129 -> 256: 5 chunks <= 8
    assert oracle.chunk_len(5, 32) == 1


@pytest.mark.parametrize("dist", ["normal", "clustered", "discrete"])
def test_chunked_with_windows_covering_chunks_is_exact(dist):
    """When k >= the chunk length every window is its whole chunk, so the candidates are all
    j <= i and the chunked search returns the exact selection."""
    w = inputs.Workload("t", 1, 2, 256, 8, 32, dist=dist, seed=14)
    x = inputs.make_inputs(w)
    zq, zk = oracle.encode(x["q"]), oracle.encode(x["k"])
    exact = oracle.select_codes(zq, zk, w.N, w.topk)
    for C in (8, 16, 32):   # chunk lengths 32, 16, 8 <= k
        np.testing.assert_array_equal(oracle.select_chunked(zq, zk, w.N, w.topk, C), exact)


def _chunked_brute(zq, zk, N, K, C, bh, i):
    """numpy form of the chunked reading for one query (candidates by window)."""
    L = 1
    while L * C < N:
        L *= 2
    cands = []
    for c in range(i // L + 1):
        lo, hi = c * L, min(N, (c + 1) * L)
        ent = sorted((int(zk[bh * N + j]), j) for j in range(lo, hi))
        n = len(ent)
        p = sum(1 for code, _ in ent if code < int(zq[bh * N + i]))
        wdt = min(K, n)
        w0 = min(max(p - K // 2, 0), n - wdt)
        cands += [(abs(int(zq[bh * N + i]) - code), j) for code, j in ent[w0:w0 + wdt] if j <= i]
    sel = [j for _, j in sorted(cands)[:K]]
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("N,K,C", [(100, 5, 4), (257, 8, 8), (64, 3, 32), (300, 16, 4)])
def test_chunked_matches_numpy_reading(N, K, C):
    w = inputs.Workload("t", 1, 2, N, 8, K, dist="clustered", seed=N + K + C)
    x = inputs.make_inputs(w)
    zq, zk = oracle.encode(x["q"]).reshape(-1), oracle.encode(x["k"]).reshape(-1)
    idx = oracle.select_chunked(zq, zk, N, K, C)
    rng = np.random.default_rng(0)
    for row in list(rng.integers(0, 2 * N, 60)) + [0, N - 1, N, 2 * N - 1]:
        bh, i = divmod(int(row), N)
        assert idx[row].tolist() == _chunked_brute(zq, zk, N, K, C, bh, i), (row,)


def test_chunked_results_are_causal_sorted_distinct():
    w = inputs.Workload("t", 1, 2, 400, 8, 24, dist="normal", seed=15)
    x = inputs.make_inputs(w)
    zq, zk = oracle.encode(x["q"]).reshape(2, -1), oracle.encode(x["k"]).reshape(2, -1)
    idx = oracle.select_chunked(zq, zk, w.N, w.topk, 8).reshape(2, w.N, -1)
    for bh in range(2):
        for i in range(w.N):
            sel = [j for j in idx[bh, i] if j >= 0]
            assert all(j <= i for j in sel) and len(set(sel)) == len(sel)
            keys = [(abs(int(zq[bh, i]) - int(zk[bh, j])), j) for j in sel]
            assert keys == sorted(keys)
            assert all(j == -1 for j in idx[bh, i, len(sel):])


# --------------------------------------------------------------------------- several curves
def test_multi_curve_equal_coordinates_is_one_curve():
    """When every point has three equal coordinates, all curves give the same codes, so the
    merged selection is the exact top-(k // P) followed by -1."""
    w = inputs.Workload("t", 1, 1, 120, 8, 18, dist="normal", seed=16)
    x = inputs.make_inputs(w)
    q = np.repeat(x["q"][..., :1], 3, axis=-1)
    k = np.repeat(x["k"][..., :1], 3, axis=-1)
    for bits in (10, 12):
        for P in (3, 6):
            per = w.topk // P
            idx = oracle.select_multi(q, k, w.topk, P, bits=bits)
            exact = oracle.select_ex(q, k, per, bits)
            np.testing.assert_array_equal(idx[:, :per], exact)
            assert np.all(idx[:, per:] == -1)


def test_chunked_on_12_bit_codes_reduces_to_exact():
    w = inputs.Workload("t", 1, 2, 200, 8, 16, dist="clustered", seed=23)
    x = inputs.make_inputs(w)
    zq, zk = oracle.encode_ex(x["q"], 12), oracle.encode_ex(x["k"], 12)
    np.testing.assert_array_equal(oracle.select_chunked(zq, zk, w.N, w.topk, 16),
                                  oracle.select_codes64(zq, zk, w.N, w.topk))


@pytest.mark.parametrize("P", [3, 6])
def test_multi_curve_union_of_per_curve_selections(P):
    w = inputs.Workload("t", 1, 2, 150, 8, 12, dist="clustered", seed=17)
    x = inputs.make_inputs(w)
    per = w.topk // P
    perms = ([(0, 1, 2), (1, 2, 0), (2, 0, 1)] if P == 3 else
             [(0, 1, 2), (0, 2, 1), (1, 2, 0), (1, 0, 2), (2, 0, 1), (2, 1, 0)])
    curves = [oracle.select_codes64(oracle.encode_ex(x["q"], 10, p), oracle.encode_ex(x["k"], 10, p),
                                    w.N, per) for p in perms]
    idx = oracle.select_multi(x["q"], x["k"], w.topk, P)
    for row in range(idx.shape[0]):
        want = []
        for c in curves:
            for j in c[row]:
                if j >= 0 and j not in want:
                    want.append(int(j))
        got = [int(j) for j in idx[row] if j >= 0]
        assert got == want, row
        assert np.all(idx[row, len(got):] == -1)


# --------------------------------------------------------------------------- Euclidean top-k
def test_euclid_topk_brute_force():
    rng = np.random.default_rng(18)
    q = rng.normal(0, 1, (1, 1, 60, 3)).astype(np.float32)
    k = rng.normal(0, 1, (1, 1, 60, 3)).astype(np.float32)
    for causal in (True, False):
        idx = oracle.euclid_topk(q, k, 5, causal)
        for i in range(60):
            n = i + 1 if causal else 60
            d = ((q[0, 0, i].astype(np.float64) - k[0, 0, :n].astype(np.float64)) ** 2).sum(-1)
            want = sorted(range(n), key=lambda j: (d[j], j))[:5]
            assert idx[i, :len(want)].tolist() == want


def test_euclid_topk_hand_example():
    # keys on the first axis at 3, 1, 2, 1 (two ties at distance 1: smaller j first)
    k = np.array([[3, 0, 0], [1, 0, 0], [2, 0, 0], [-1, 0, 0]], dtype=np.float32)[None, None]
    q = np.zeros((1, 1, 4, 3), dtype=np.float32)
    idx = oracle.euclid_topk(q, k, 3, causal=False)
    np.testing.assert_array_equal(idx, np.tile([1, 3, 2], (4, 1)))


# --------------------------------------------------------------------------- empty selection
def test_empty_selection_gives_zero_output_and_no_gradient():
    w = inputs.Workload("t", 1, 1, 6, 8, 3, dist="normal", seed=19)
    x = inputs.make_inputs(w)
    idx = oracle.select(x["q"], x["k"], w.topk)
    idx[2] = -1  # query 2 selects nothing
    out = oracle.forward(x["q"], x["k"], x["v"], x["gamma"], idx, False)
    assert np.all(out[2] == 0.0) and np.all(np.isfinite(out))
    dout = np.ones((1, 1, 6, 8), dtype=np.float32)
    dq, dk, dv, dg = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], dout, idx, False)
    assert np.all(dq[2] == 0.0)
    # removing query 2's row from the list changes nothing else
    rows = np.array([0, 1, 3, 4, 5])
    dq2, dk2, dv2, dg2 = oracle.backward(x["q"], x["k"], x["v"], x["gamma"], dout, idx[rows],
                                         False, rows=rows)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
    np.testing.assert_array_equal(dg, dg2)
