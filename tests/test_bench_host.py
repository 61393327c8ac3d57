"""Host-side logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte model
against closed forms, and the parsers of the rocprofv3 outputs it summarises."""

import csv
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from order_retrieval_amd import inputs  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused_with_a_message(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _sum_valid_slots(N, k):
    # sum over i < N of min(k, i + 1), written out: 1 + 2 + ... + k for the first k queries,
    # then k for each of the remaining N - k
    if N <= k:
        return N * (N + 1) // 2
    return k * (k + 1) // 2 + k * (N - k)


def test_gather_bytes_closed_form():
    w = inputs.CONFIGS["long_fwd_bwd"]
    row = w.dv * (2 if w.v_dtype == inputs.BF16 else 4)
    BH = w.B * w.H
    # per query: 4m + 12 + 12m + m row + row -- index, key row and value row of each of the m
    # selected slots, the query point and the output row
    want = BH * (_sum_valid_slots(w.N, w.topk) * (16 + row) + w.N * (12 + row))
    assert bench.algorithmic_bytes(w)["gather"] == pytest.approx(want, rel=0, abs=0.5)


@pytest.mark.parametrize("name,fwd_mb", [("tiny", 10.5), ("multihead", 354), ("clustered", 11400),
                                         ("long_fwd", 6280)])
def test_forward_bytes_match_the_scope_table(name, fwd_mb):
    # the forward totals of the method's byte model (encode + sort + select + gather), as
    # tabulated per configuration: 10.5 MB, 354 MB, 11.40 GB, 6.28 GB (the table counts k
    # slots for every query, the model here m = min(k, i+1): 1.4 % fewer bytes at N = 1024)
    b = bench.algorithmic_bytes(inputs.CONFIGS[name])
    got = (b["encode_order"] - 12 * inputs.CONFIGS[name].rows + b["tree"] + b["select"] +
           b["gather"]) / 1e6
    assert got == pytest.approx(fwd_mb, rel=0.02)


@pytest.mark.parametrize("N,k,want", [(65536, 32, 10), (16384, 64, 7), (1024, 32, 4),
                                      (1000, 64, 3), (100, 64, 0), (65536, 256, 7),
                                      (64, 32, 1), (128, 32, 1), (129, 32, 2)])
def test_stored_levels(N, k, want):
    w = inputs.Workload("s", 1, 1, N, 8, k)
    assert bench.stored_levels(w) == want


def _count_bit_set(n, l):
    """How many m in [1, n] have bit l set (the standard block count)."""
    block = 1 << (l + 1)
    full = (n + 1) // block
    rest = (n + 1) % block
    return full * (1 << l) + max(0, rest - (1 << l))


@pytest.mark.parametrize("name", ["tiny", "multihead", "long_fwd"])
def test_select_bytes_closed_form(name):
    w = inputs.CONFIGS[name]
    k = w.topk
    want = 0.0
    for l in range(w.N.bit_length()):
        want += _count_bit_set(w.N, l) * (8.0 * (l + 1) + 8.0 * min(2 * k, 1 << l))
    want += w.N * (4 + 4 * k)
    got = bench.variant_select_bytes(w, "exact") / (w.B * w.H)
    assert got == pytest.approx(want, rel=1e-12)


def test_kernel_base_names():
    assert bench.kernel_base("void zeta::zeta_select_kernel<32, 4, unsigned int, 32, true>"
                             "(unsigned int const*, unsigned int const*)") == "zeta_select_kernel"
    assert bench.kernel_base("zeta::zeta_tree_merge_kernel(unsigned long*, long)") == \
        "zeta_tree_merge_kernel"


def _write_csv(path, header, rows):
    # quoted where needed, as rocprofv3 writes kernel names that hold commas
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_counter_means_average_per_dispatch(tmp_path):
    _write_csv(tmp_path / "x_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["void zeta::zeta_bwd_key_kernel<true, true, 1>(float const*)", "FETCH_SIZE", 100],
                ["void zeta::zeta_bwd_key_kernel<true, true, 1>(float const*)", "FETCH_SIZE", 300],
                ["zeta::zeta_morton_encode_kernel(float const*)", "FETCH_SIZE", 7],
                ["zeta::zeta_morton_encode_kernel(float const*)", "WRITE_SIZE", 9]])
    m = bench.counter_means(str(tmp_path), "FETCH_SIZE")
    assert m == {"zeta_bwd_key_kernel": 200.0, "zeta_morton_encode_kernel": 7.0}


def test_trace_kernels_average_duration(tmp_path):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "VGPR_Count", "Accum_VGPR_Count",
           "LDS_Block_Size", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]
    _write_csv(tmp_path / "tr_kernel_trace.csv", hdr,
               [["zeta::zeta_select_kernel<32>(int)", 1000, 5000, 32, 0, 0, 256, 1, 1],
                ["zeta::zeta_select_kernel<32>(int)", 9000, 15000, 32, 0, 0, 256, 1, 1]])
    t = bench.trace_kernels(str(tmp_path))
    assert t["zeta_select_kernel"]["n"] == 2
    assert t["zeta_select_kernel"]["us"] == pytest.approx(5.0)  # (4000 + 6000) ns / 2
    assert t["zeta_select_kernel"]["wg"] == 256


@pytest.mark.parametrize("lds,wg,want", [(0, 256, 8), (39424, 256, 4), (32768, 1024, 8),
                                         (163840, 1024, 4), (81920, 256, 2)])
def test_waves_allowed_by_lds(lds, wg, want):
    assert bench.waves_by_lds(lds, wg) == want


def test_stored_traffic_is_dropped_when_the_source_changed(tmp_path, monkeypatch):
    src_dir = tmp_path / "order_retrieval_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "gather.hip"
    src.write_bytes(b"kernel v1")
    rec = {"source_sha256": hashlib.sha256(b"kernel v1").hexdigest(), "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "gather_long_fwd_bwd_counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("gather") == 123
    src.write_bytes(b"kernel v2")
    assert bench.stored_traffic("gather") is None
