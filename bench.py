#!/usr/bin/env python3
"""Benchmark of the ZETA causal top-k attention hot path on one MI355X.

A step is one zeta_fwd (encode, tree build, select, Cauchy gather) plus one zeta_bwd
(per-query pass, selection transpose, per-key pass, dgamma) on the 65536-token workload
B=1, H=8, N=65536, d_K=3, d_V=128, k=32 with bf16 v and dO (seeded synthetic inputs,
already resident in HBM when the timed region starts).  Prints one JSON line.

Kernel durations come from HIP events that the library records on its launch stream
between stages (zeta_set_stage_events), inside the timed steps.  The CPU baseline is the
oracle timed on a bounded random sample of query rows and scaled to the full step.
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from order_retrieval_amd import inputs  # noqa: E402

METRIC = "ms per ZETA fwd (and fwd+bwd) at N=65536,H=8; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PAGES_CONTEXT = {"zeta_fwd_ms": 85.8, "zeta_fwd_bwd_ms": 608.2, "flash_fwd_ms": 805.3,
                 "flash_fwd_bwd_ms": 7044.1, "hardware": "not stated on the pages"}
FWD_STAGES = ["encode_order", "tree", "select", "order", "gather"]
BWD_STAGES = ["bwd_order", "bwd_query", "bwd_transpose", "bwd_key", "bwd_dgamma"]
SINGLE_KERNEL = {"select": "zeta_select_kernel", "gather": "zeta_cauchy_gather_kernel",
                 "bwd_query": "zeta_bwd_query_kernel", "bwd_key": "zeta_bwd_key_kernel"}
KERNEL_SOURCE = {"select": "select.hip", "gather": "gather.hip", "bwd_query": "backward.hip",
                 "bwd_key": "backward.hip"}


# ----------------------------------------------------------------------------- bytes
def valid_slots(w: inputs.Workload) -> np.ndarray:
    """m_i = min(k, i+1): selected keys of query i (same for every (b,h))."""
    return np.minimum(np.arange(w.N, dtype=np.int64) + 1, w.topk)


def select_run_bytes(w: inputs.Workload) -> float:
    """Per (b,h): for every query, the sorted runs of its causal prefix (set bits of i+1):
    a binary search (floor(log2 s)+1 probes of 8 B) and two k-wide windows (<= s entries of
    8 B) per run, plus the query code (4 B) and the written index row (4k B)."""
    i1 = np.arange(1, w.N + 1, dtype=np.int64)
    total = np.zeros(w.N, dtype=np.float64)
    for l in range(int(np.log2(w.N)) + 1):
        s = 1 << l
        has = (i1 >> l) & 1
        total += has * (8.0 * (l + 1) + 8.0 * min(2 * w.topk, s))
    return float((total + 4 + 4 * w.topk).sum())


def variant_select_bytes(w: inputs.Workload, mode: str, causal: bool = True, chunks: int = 0,
                         curves: int = 0, bits: int = 10) -> float:
    """Algorithmic bytes of one selection launch (all (b,h)) of a variant, counted as for
    the exact selection: 8 B per tree entry probed or windowed, the query code, idx out."""
    BH, N, k = w.B * w.H, w.N, w.topk
    zb = 8 if bits == 12 else 4
    if mode == "exact":
        m = np.arange(1, N + 1, dtype=np.int64) if causal else np.full(N, N, dtype=np.int64)
        total = np.zeros(N, dtype=np.float64)
        for l in range(int(np.log2(N)) + 1):
            s = 1 << l
            total += ((m >> l) & 1) * (8.0 * (l + 1) + 8.0 * min(2 * k, s))
        return BH * float((total + zb + 4 * k).sum())
    if mode == "chunked":
        L = 1
        while L * chunks < N:
            L *= 2
        lvl = int(np.log2(L))
        nch = np.arange(N, dtype=np.int64) // L + 1  # chunks searched by query i
        per = 8.0 * (lvl + 1) + 8.0 * min(k, L)
        return BH * float((nch * per + zb + 4 * k).sum())
    per = k // curves  # several curves: exact selections of k // P, then the merge
    sub = inputs.Workload(**{**w.__dict__, "topk": per})
    one = variant_select_bytes(sub, "exact", causal, bits=bits)
    return curves * one + BH * N * (curves * per * 4 + 4 * k)


VARIANTS = [  # name, zeta_select_opts fields
    ("exact_noncausal", dict(mode=0, causal=False)),
    ("exact_12bit", dict(mode=0, causal=True, bits=12)),
    ("chunked_4", dict(mode=1, chunks=4)),
    ("chunked_8", dict(mode=1, chunks=8)),
    ("chunked_16", dict(mode=1, chunks=16)),
    ("chunked_32", dict(mode=1, chunks=32)),
    ("curves_3", dict(mode=2, curves=3)),
    ("curves_6", dict(mode=2, curves=6)),
]


def kernel_bytes(w: inputs.Workload) -> dict:
    """Algorithmic bytes per launch of each kernel (every gathered row counted as read)."""
    BH = w.B * w.H
    vb = 2 if w.v_dtype == inputs.BF16 else 4
    row = w.dv * vb
    m = valid_slots(w).astype(np.float64)
    pairs = float(m.sum())  # per (b,h)
    levels = int(np.log2(w.N)) + 1
    tile_levels = min(levels - 1, 10)
    b = {}
    # encode of q and k, then the query processing order (codes counted, codes placed,
    # order written), which the select and the gather both use
    b["encode_order"] = BH * w.N * (2 * 12 + 2 * 4) + BH * w.N * (4 + 4 + 4)
    b["tree"] = BH * w.N * (4 + 2 * 8 * (tile_levels + 1) + 2 * 16 * (levels - 1 - tile_levels))
    b["select"] = BH * select_run_bytes(w)
    b["order"] = 0  # built with the encodes on this path
    b["gather"] = BH * float((4 * m + 12 + 12 * m + m * row + 4 + row).sum())
    b["bwd_order"] = BH * w.N * (2 * 12 + 2 * 4 + 2 * 12)
    # per query: index row, q, key rows, value rows, dO row, dq and dgamma term, processing
    # order entry, and {a, c} of every selected slot
    b["bwd_query"] = BH * float((4 * m + 12 + 12 * m + m * row + row + 16 + 4 + 8 * m).sum())
    bits = int(np.ceil(np.log2(w.N))) if w.N > 1 else 0
    # pass 0 reads the index rows twice (histogram, scatter) and writes 8-byte {j, p} records;
    # keys below 2^16: the per-group sort reads the records twice (count, scatter) and writes
    # 4-byte slots and two segment bounds per key; wider keys: every further pass reads the
    # records twice and writes them, and the segment starts read the sorted records
    if bits <= 16:
        b["bwd_transpose"] = BH * (2 * 4 * w.N * w.topk + 8 * pairs + 16 * pairs + 4 * pairs +
                                   8 * w.N)
    else:
        passes = -(-bits // 8)
        b["bwd_transpose"] = BH * (2 * 4 * w.N * w.topk + 8 * pairs + (passes - 1) * 24 * pairs +
                                   8 * pairs + 4 * (w.N + 1))
    # per key: gamma, two offsets, k, dk and its dv row; per pair: the record, {a, c}, q_i
    # and the dO_i row
    b["bwd_key"] = BH * (w.N * (4 + 8 + 12 + 12 + row) + pairs * (8 + 8 + 12 + row))
    b["bwd_dgamma"] = BH * w.N * 4.0
    return b


# ----------------------------------------------------------------------------- HIP events
class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded (shared with libzeta)."""

    def __init__(self, runtime_path: str):
        self.lib = ctypes.CDLL(runtime_path)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        evs = (ctypes.c_void_p * n)()
        for t in range(n):
            h = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            evs[t] = h
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, evs):
        for h in evs:
            self.lib.hipEventDestroy(h)


# ----------------------------------------------------------------------------- counters
def stored_traffic(stage: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/*_counters.json), used
    only while the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_long_fwd_bwd_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "order_retrieval_amd", "csrc", KERNEL_SOURCE[stage])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- reports
def kernel_base(name: str) -> str:
    """zeta::zeta_select_kernel<32, 2>(...) -> zeta_select_kernel."""
    base = name.split("(")[0].split("<")[0]
    return base.replace("void ", "").split("::")[-1].strip()


def counter_means(path: str, counter: str) -> dict:
    """Mean counter value per dispatch of each kernel in a rocprofv3 --pmc csv output dir."""
    files = glob.glob(os.path.join(path, "*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    vals: dict = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(kernel_base(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


COUNTER_CMDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o fetch -- "
    "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-variants",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o write -- "
    "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-variants",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_fetch -o copy_fetch -- "
    "python3 bench.py --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_write -o copy_write -- "
    "python3 bench.py --copy-calibration",
    "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_WAVES SQ_WAVE_CYCLES "
    "SQ_BUSY_CYCLES --output-format csv -d {d}/lds -o lds -- "
    "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-variants",
]
# sort and select stages, whose LDS use and occupancy the counters report
SORT_SELECT = ("zeta_order_", "zeta_tree_", "zeta_radix_", "zeta_bucket_sort", "zeta_select_")
CU_COUNT, SIMDS_PER_CU, CLOCK_GHZ, LDS_BYTES_PER_CU = 256, 4, 2.4, 160 * 1024


def trace_kernels(d: str) -> dict:
    """Per kernel (base name): average duration (us) and resources from a kernel trace dir."""
    out: dict = {}
    for f in glob.glob(os.path.join(d, "*kernel_trace.csv")):
        for r in csv.DictReader(open(f)):
            k = kernel_base(r["Kernel_Name"])
            e = out.setdefault(k, {"n": 0, "ns": 0.0})
            e["n"] += 1
            e["ns"] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            e.update(vgpr=int(r["VGPR_Count"]) + int(r["Accum_VGPR_Count"]),
                     lds=int(r["LDS_Block_Size"]), wg=int(r["Workgroup_Size_X"]) *
                     int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
    for e in out.values():
        e["us"] = e["ns"] / e["n"] / 1e3
    return out


def waves_by_lds(lds: int, wg: int) -> int:
    """Resident wavefronts per SIMD that a workgroup's LDS allows (160 KiB per CU, 4 SIMDs,
    at most 8 wavefronts per SIMD)."""
    waves_wg = -(-wg // 64)
    wgs = LDS_BYTES_PER_CU // lds if lds > 0 else 64
    return min(8, (wgs * waves_wg) // SIMDS_PER_CU)
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o tr -- "
             "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-variants")


def counters_summary(d: str, workload: str) -> None:
    """HBM bytes per launch of the hot kernels from FETCH_SIZE / WRITE_SIZE passes, each scaled
    by what the same counter reads for a plain 1 GiB device copy; writes
    profiles/<stage>_<workload>_counters.json (keyed to the kernel source's sha256) and a
    markdown table of every kernel."""
    copy_bytes = float(1 << 30)
    cf = counter_means(os.path.join(d, "copy_fetch"), "FETCH_SIZE")
    cw = counter_means(os.path.join(d, "copy_write"), "WRITE_SIZE")
    copy_name = next(k for k in cf if "copyBuffer" in k or "copy" in k.lower())
    fscale = copy_bytes / (cf[copy_name] * 1024.0)
    wscale = copy_bytes / (cw[copy_name] * 1024.0)
    fetch = counter_means(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = counter_means(os.path.join(d, "write"), "WRITE_SIZE")
    cmds = [c.format(d=d) for c in COUNTER_CMDS]
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    lines = [f"# HBM traffic per launch, {workload} (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (each pass its own run, from the repository root):", ""]
    lines += [f"    {c}" for c in cmds] + [f"    python3 bench.py --counters-summary {d}", ""]
    lines += [f"Copy calibration: a 1 GiB device copy reads {cf[copy_name]:.0f} KiB (FETCH_SIZE) and "
              f"writes {cw[copy_name]:.0f} KiB (WRITE_SIZE): scale {fscale:.3f} and {wscale:.3f}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB per launch (scaled) |",
              "|---|---|---|---|"]
    for kname in sorted(fetch, key=lambda n: -fetch[n]):
        if not kname.startswith("zeta_"):
            continue
        hb = fetch[kname] * 1024 * fscale + write.get(kname, 0.0) * 1024 * wscale
        lines.append(f"| {kname} | {fetch[kname]:.0f} | {write.get(kname, 0.0):.0f} | {hb / 1e6:.1f} |")
    for stage, kname in SINGLE_KERNEL.items():
        if kname not in fetch:
            continue
        src = os.path.join(ROOT, "order_retrieval_amd", "csrc", KERNEL_SOURCE[stage])
        rec = {"kernel": kname, "workload": workload,
               "fetch_kib": fetch[kname], "write_kib": write.get(kname, 0.0),
               "fetch_scale": fscale, "write_scale": wscale,
               "hbm_bytes_per_launch": int(fetch[kname] * 1024 * fscale +
                                           write.get(kname, 0.0) * 1024 * wscale),
               "source": KERNEL_SOURCE[stage],
               "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
               "commands": cmds}
        with open(os.path.join(prof, f"{stage}_{workload}_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
    tr = os.path.join(os.path.dirname(os.path.abspath(d)), "trace")
    kt = trace_kernels(tr) if os.path.isdir(tr) else {}
    if kt:
        lines += ["", f"Achieved HBM rate: the bytes above over the average kernel duration of the "
                  f"kernel trace in {tr} (the same bench command, its own run):", "",
                  "| kernel | HBM MB per launch | average us | HBM GB/s | of 8 TB/s |", "|---|---|---|---|---|"]
        for kname in sorted(fetch, key=lambda n: -fetch[n]):
            if not kname.startswith("zeta_") or kname not in kt:
                continue
            hb = fetch[kname] * 1024 * fscale + write.get(kname, 0.0) * 1024 * wscale
            gbs = hb / (kt[kname]["us"] * 1e-6) / 1e9
            lines.append(f"| {kname} | {hb / 1e6:.1f} | {kt[kname]['us']:.1f} | {gbs:.0f} | "
                         f"{gbs / HBM_PEAK_GBS:.1%} |")
    ldsdir = os.path.join(d, "lds")
    if os.path.isdir(ldsdir) and kt:
        m = {c: counter_means(ldsdir, c) for c in ("SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
                                                   "SQ_INSTS_LDS", "SQ_WAVES", "SQ_WAVE_CYCLES")}
        lines += ["", "Sort and select stages: LDS bank conflicts and occupancy (one counter pass "
                  "with SQ_LDS_BANK_CONFLICT, SQ_ACTIVE_INST_LDS, SQ_INSTS_LDS, SQ_WAVES, "
                  "SQ_WAVE_CYCLES, SQ_BUSY_CYCLES; workgroup size, LDS bytes and the VGPR_Count "
                  "field as the kernel trace records them).  \"conflict cycles per LDS "
                  "instruction\" is SQ_LDS_BANK_CONFLICT over SQ_INSTS_LDS (wavefront "
                  "instructions); \"waves/SIMD (LDS)\" is the residency the workgroup's LDS allows "
                  "(160 KiB per CU, at most 8); \"waves/SIMD mean\" is SQ_WAVE_CYCLES (counted in "
                  "4-cycle units) over the SIMDs' cycles of the average duration.", "",
                  "| kernel | LDS instructions | bank-conflict cycles | conflict cycles per LDS "
                  "instruction | VGPR_Count (trace) | LDS bytes | workgroup | waves/SIMD (LDS) | "
                  "waves/SIMD mean |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for kname in sorted(kt, key=lambda n: -kt[n]["us"]):
            if not kname.startswith(SORT_SELECT) or kname not in m["SQ_WAVES"]:
                continue
            e = kt[kname]
            ninst = m["SQ_INSTS_LDS"].get(kname, 0.0)
            conf = m["SQ_LDS_BANK_CONFLICT"].get(kname, 0.0)
            share = f"{conf / ninst:.2f}" if ninst > 0 else "-"
            mean = 4 * m["SQ_WAVE_CYCLES"][kname] / (CU_COUNT * SIMDS_PER_CU * e["us"] * 1e3 *
                                                      CLOCK_GHZ)
            lines.append(f"| {kname} | {m['SQ_INSTS_LDS'].get(kname, 0.0):.0f} | {conf:.0f} | "
                         f"{share} | {e['vgpr']} | {e['lds']} | {e['wg']} | "
                         f"{waves_by_lds(e['lds'], e['wg'])} | {mean:.1f} |")
    with open(os.path.join(prof, f"counters_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def trace_summary(d: str, workload: str) -> None:
    """Per-kernel durations from a rocprofv3 --kernel-trace --stats run, next to the bench line
    the same run printed (its stage_ms come from HIP events on the launch stream)."""
    stats = glob.glob(os.path.join(d, "*kernel_stats.csv"))
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(stats[0])))
    bench_line = None
    log = os.path.join(d, "run.log")
    if os.path.exists(log):
        for ln in open(log):
            if ln.startswith("{"):
                bench_line = json.loads(ln)
    lines = [f"# Kernel durations, {workload} (rocprofv3 --kernel-trace --stats)", "",
             "Command (from the repository root; stdout to run.log in the same folder):", "",
             f"    {TRACE_CMD.format(d=d)}", f"    python3 bench.py --trace-summary {d}", "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    if bench_line is not None:
        lines += ["", "Stage times the same run measured with HIP events (ms per launch):", "",
                  "    " + json.dumps(bench_line["stage_ms"]),
                  "", f"fwd+bwd step: {bench_line['value']} ms; roofline: "
                  + json.dumps(bench_line["roofline"])]
    with open(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


# ----------------------------------------------------------------------------- variants
def _recall(sel, ref, torch) -> float:
    """Mean over queries of |sel & ref| / |ref| (valid entries only)."""
    hit = (sel.unsqueeze(-1) == ref.unsqueeze(-2)) & (ref >= 0).unsqueeze(-2)
    found = hit.any(dim=-2).sum(dim=-1).double()
    want = (ref >= 0).sum(dim=-1).double()
    keep = want > 0
    return float((found[keep] / want[keep]).mean().item())


def _euclid_topk(q, k, rows, topk, causal, torch):
    """Exact Euclidean top-k (by squared distance, ties to the smaller j) of sampled queries
    of every head, brute force in fp64 on the device: [BH, S, topk] (-1 padded)."""
    BH, N = q.shape[0] * q.shape[1], q.shape[2]
    qf = q.reshape(BH, N, 3).double()
    kf = k.reshape(BH, N, 3).double()
    out = torch.full((BH, rows.numel(), topk), -1, dtype=torch.int32, device=q.device)
    j = torch.arange(N, device=q.device)
    for bh in range(BH):
        d = ((qf[bh, rows].unsqueeze(1) - kf[bh].unsqueeze(0)) ** 2).sum(-1)  # [S, N]
        if causal:
            d = d.masked_fill(j.unsqueeze(0) > rows.unsqueeze(1), float("inf"))
        # ties to the smaller j: a stable sort of the distances
        order = torch.sort(d, dim=1, stable=True).indices[:, :topk]
        valid = torch.gather(d, 1, order) < float("inf")
        out[bh] = torch.where(valid, order, torch.full_like(order, -1)).to(torch.int32)
    return out


def measure_variants(w, q, k, v, gamma, dout, idx_exact, hip, lib, Z, torch, steps: int) -> dict:
    """Each selection variant: stage times of zeta_fwd_ex (select = encode + tree + select
    stages) and of zeta_bwd_ex, the select kernel's algorithmic bytes per second, and the
    recall of its selection against the exact causal one and against the exact Euclidean
    top-k (sampled queries).  Recall is computed outside the timed region."""
    res = {}
    BH, N, K = w.B * w.H, w.N, w.topk
    g = torch.Generator(device="cpu").manual_seed(1234)
    rows = torch.randint(0, N, (256,), generator=g).to(q.device)
    exact_rows = idx_exact.reshape(BH, N, K)[:, rows]
    eu_causal = _euclid_topk(q, k, rows, K, True, torch)
    eu_all = _euclid_topk(q, k, rows, K, False, torch)
    res["exact_causal"] = {"recall_vs_euclidean": round(_recall(exact_rows, eu_causal, torch), 4)}
    out = torch.empty_like(v)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((w.H,), dtype=torch.float32, device=q.device))
    shape = Z.make_shape(w.B, w.H, N, w.dv, K, Z.ZETA_BF16 if v.dtype == torch.bfloat16 else Z.ZETA_F32)
    for name, f in VARIANTS:
        o = Z.select_opts(f.get("mode", 0), causal=f.get("causal", True), bits=f.get("bits", 10),
                          chunks=f.get("chunks", 0), curves=f.get("curves", 0))
        ws_f = Z.workspace(shape, Z.ZETA_WS_FWD, q.device, o)
        ws_b = Z.workspace(shape, Z.ZETA_WS_BWD, q.device, o)
        idx = torch.empty((w.B, w.H, N, K), dtype=torch.int32, device=q.device)
        for _ in range(2):
            Z.zeta_fwd_ex(q, k, v, gamma, K, o, ws=ws_f, out=out, idx=idx)
            Z.zeta_bwd_ex(q, k, v, gamma, idx, dout, o, ws=ws_b, grads=grads)
        ev = [(hip.create(6), hip.create(6)) for _ in range(steps)]
        torch.cuda.synchronize()
        for ef, eb in ev:
            lib.zeta_set_stage_events(ef, 6)
            Z.zeta_fwd_ex(q, k, v, gamma, K, o, ws=ws_f, out=out, idx=idx)
            lib.zeta_set_stage_events(eb, 6)
            Z.zeta_bwd_ex(q, k, v, gamma, idx, dout, o, ws=ws_b, grads=grads)
            lib.zeta_set_stage_events(None, 0)
        torch.cuda.synchronize()
        sel = float(np.mean([hip.elapsed_ms(ef[0], ef[3]) for ef, _ in ev]))
        sel_k = float(np.mean([hip.elapsed_ms(ef[2], ef[3]) for ef, _ in ev]))
        fwd = float(np.mean([hip.elapsed_ms(ef[0], ef[5]) for ef, _ in ev]))
        bwd = float(np.mean([hip.elapsed_ms(eb[0], eb[5]) for _, eb in ev]))
        for ef, eb in ev:
            hip.destroy(ef)
            hip.destroy(eb)
        mode = ["exact", "chunked", "curves"][f.get("mode", 0)]
        sb = variant_select_bytes(w, mode, f.get("causal", True), f.get("chunks", 0),
                                  f.get("curves", 0), f.get("bits", 10))
        sel_rows = idx.reshape(BH, N, K)[:, rows]
        r = {"select_stages_ms": round(sel, 4), "select_kernel_ms": round(sel_k, 4),
             "fwd_ms": round(fwd, 4), "fwd_bwd_ms": round(fwd + bwd, 4),
             "select_algorithmic_GBs": round(sb / ((sel if mode == "curves" else sel_k) * 1e-3)
                                             / 1e9, 1),
             "recall_vs_exact_causal": round(_recall(sel_rows, exact_rows, torch), 4),
             "recall_vs_euclidean": round(_recall(sel_rows, eu_causal if f.get("causal", True)
                                                  else eu_all, torch), 4)}
        if mode == "curves":  # stage 3 spans the later curves and the merge
            r["note"] = "select_kernel_ms covers curves 2..P and the merge; GB/s over all stages"
        res[name] = r
        del ws_f, ws_b
    return res


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(w: inputs.Workload, x: dict, target_s: float, seed: int = 0) -> dict:
    import oracle

    bf = w.v_dtype == inputs.BF16
    total = w.B * w.H * w.N
    rng = np.random.default_rng(seed)

    def run(count):
        rows = np.sort(rng.choice(total, size=count, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        idx = oracle.select(x["q"], x["k"], w.topk, rows=rows)
        oracle.forward(x["q"], x["k"], x["v"], x["gamma"], idx, bf, rows=rows)
        oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["dout"], idx, bf, rows=rows)
        return time.perf_counter() - t0

    # the oracle's backward zeroes full-size dk/dv arrays on every call, so calibrate the
    # sample size from the cost difference of two probe sizes (marginal cost per row)
    p1, p2 = min(256, total), min(2048, total)
    t1, t2 = run(p1), run(p2)
    per_row = max((t2 - t1) / max(p2 - p1, 1), 1e-7)
    count = int(min(total, max(p2, (target_s - t1) / per_row)))
    t = run(count)
    return {"value": round(t / count * total * 1e3, 1), "unit": "ms", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": (f"{count} uniformly drawn query rows of the same workload (select + forward "
                       f"+ backward contributions, {t:.1f} s), scaled by {total}/{count}; "
                       f"selection and forward use all threads, backward runs on one")}


# ----------------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_fwd_bwd", choices=sorted(inputs.CONFIGS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the selection variants (chunked, several curves, unmasked, 12-bit)")
    ap.add_argument("--variant-steps", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device-to-device copies (counter calibration)")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="write profiles/*_counters.json from rocprofv3 --pmc outputs under DIR")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 kernel-trace run")
    args = ap.parse_args()
    if args.counters_summary:
        counters_summary(args.counters_summary, args.workload)
        return 0
    if args.trace_summary:
        trace_summary(args.trace_summary, args.workload)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the (b,h) slices "
              "are independent and each GPU would run this same kernel sequence on its heads.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        # known-size plain copies: the HBM counters of this kernel give the scale factor
        # between counter readings and bytes (1 GiB read + 1 GiB written per copy)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": src.numel() * 4,
                          "copies": 5}), flush=True)
        return 0

    from order_retrieval_amd import zeta as Z

    w = inputs.CONFIGS[args.workload]
    w = inputs.Workload(**{**w.__dict__, "backward": True})
    x = inputs.make_inputs(w)
    dev = torch.device("cuda", 0)
    bf = w.v_dtype == inputs.BF16

    def to_dev(a, as_bf16=False):
        if as_bf16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, gamma = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["gamma"])
    v, dout = to_dev(x["v"], bf), to_dev(x["dout"], bf)
    shape = Z.make_shape(w.B, w.H, w.N, w.dv, w.topk, Z.ZETA_BF16 if bf else Z.ZETA_F32)
    ws_f = Z.workspace(shape, Z.ZETA_WS_FWD, dev)
    ws_b = Z.workspace(shape, Z.ZETA_WS_BWD, dev)
    out = torch.empty_like(v)
    idx = torch.empty((w.B, w.H, w.N, w.topk), dtype=torch.int32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((w.H,), dtype=torch.float32, device=dev))
    lib = Z.load_library()
    torch.cuda.synchronize()
    hip = HipEvents(Z.hip_runtimes_mapped()[0])

    def step(ev_f=None, ev_b=None):
        if ev_f is not None:
            lib.zeta_set_stage_events(ev_f, len(ev_f))
        Z.zeta_fwd(q, k, v, gamma, w.topk, ws=ws_f, out=out, idx=idx)
        if ev_b is not None:
            lib.zeta_set_stage_events(ev_b, len(ev_b))
        Z.zeta_bwd(q, k, v, gamma, idx, dout, ws=ws_b, grads=grads)
        lib.zeta_set_stage_events(None, 0)

    for _ in range(args.warmup):
        step()
    ev = [(hip.create(len(FWD_STAGES) + 1), hip.create(len(BWD_STAGES) + 1))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        step(*ev[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_end) / args.steps

    stages = {n: [] for n in FWD_STAGES + BWD_STAGES}
    for evf, evb in ev:
        for s, n in enumerate(FWD_STAGES):
            stages[n].append(hip.elapsed_ms(evf[s], evf[s + 1]))
        for s, n in enumerate(BWD_STAGES):
            stages[n].append(hip.elapsed_ms(evb[s], evb[s + 1]))
    stage_ms = {n: float(np.mean(t)) for n, t in stages.items()}
    fwd_ms = sum(stage_ms[n] for n in FWD_STAGES)
    bwd_ms = sum(stage_ms[n] for n in BWD_STAGES)
    for evf, evb in ev:
        hip.destroy(evf)
        hip.destroy(evb)

    # forward alone, for the forward-only figure
    fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    fs.record()
    for _ in range(args.steps):
        Z.zeta_fwd(q, k, v, gamma, w.topk, ws=ws_f, out=out, idx=idx)
    fe.record()
    torch.cuda.synchronize()
    fwd_only_ms = fs.elapsed_time(fe) / args.steps

    kb = kernel_bytes(w)
    dom = max(SINGLE_KERNEL, key=lambda n: stage_ms[n])
    achieved = kb[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = stored_traffic(dom)
    fwd_bytes = sum(kb[n] for n in FWD_STAGES)
    step_bytes = sum(kb.values())
    rows = w.B * w.H * w.N
    result = {
        "metric": METRIC,
        "value": round(step_ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} H{w.H} N{w.N} dK3 dV{w.dv} k{w.topk}, "
                               f"v/dO {w.v_dtype}, forward+backward",
                   "B": w.B, "H": w.H, "N": w.N, "d_K": 3, "d_V": w.dv, "topk": w.topk,
                   "v_dtype": w.v_dtype, "seed": w.seed},
        "fwd_ms": round(fwd_only_ms, 4),
        "fwd_bwd_ms": round(step_ms, 4),
        "queries_per_s_fwd": round(rows / (fwd_only_ms * 1e-3), 1),
        "queries_per_s_fwd_bwd": round(rows / (step_ms * 1e-3), 1),
        "fwd_algorithmic_GBs": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
        "fwd_hbm_frac": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_GBs": round(step_bytes / ((fwd_ms + bwd_ms) * 1e-3) / 1e9, 1),
        "stage_ms": {n: round(t, 4) for n, t in stage_ms.items()},
        "stage_algorithmic_bytes": {n: int(b) for n, b in kb.items()},
        "roofline": {"bound": "hbm", "kernel": SINGLE_KERNEL[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     # measured HBM bytes over the same duration: what DRAM actually carried
                     "dram_GBs": None if traffic is None
                     else round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1),
                     "dram_frac": None if traffic is None
                     else round(traffic / (stage_ms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "wall_s_timed": round(wall, 3),
        "pages_context": PAGES_CONTEXT,
        "input_sha256": inputs.digest(x),
    }
    if not args.no_variants:
        result["variants"] = measure_variants(w, q, k, v, gamma, dout, idx, hip, lib, Z, torch,
                                              args.variant_steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
