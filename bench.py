#!/usr/bin/env python3
"""Benchmark of the ZETA causal top-k attention hot path on one MI355X.

A step is one zeta_fwd (encode, tree build, select, Cauchy gather) plus one zeta_bwd
(per-query pass, selection transpose, per-key pass, dgamma) on the 65536-token workload
B=1, H=8, N=65536, d_K=3, d_V=128, k=32 with bf16 v and dO (seeded synthetic inputs,
already resident in HBM when the timed region starts).  Prints one JSON line: that step,
the same measurement for every other synthetic configuration, the memory footprint, the
measured row-gather ceiling that bounds the row kernels, and the oracle's CPU time.

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
# kernels whose time goes to gathering whole rows named by the selection (mostly L2 hits):
# bounded by the rate of such gathers (zeta_probe_row_gather), not by HBM bandwidth
ROW_KERNELS = ("gather", "bwd_query", "bwd_key")
# the row-gather ceiling: tables of 256-byte rows (one bf16 row of dV = 128)
CEILING_TABLES = [("l2_2MiB", 2 << 20), ("mall_16MiB", 16 << 20), ("hbm_1GiB", 1 << 30)]
CEILING_ROW_BYTES, CEILING_GROUPS, CEILING_ROWS = 256, 1 << 19, 32
KERNEL_SOURCE = {"select": "select.hip", "gather": "gather.hip", "bwd_query": "backward.hip",
                 "bwd_key": "backward.hip"}


# ----------------------------------------------------------------------------- bytes
def valid_slots(w: inputs.Workload) -> np.ndarray:
    """m_i = min(k, i+1): selected keys of query i (same for every (b,h))."""
    return np.minimum(np.arange(w.N, dtype=np.int64) + 1, w.topk)


def variant_select_bytes(w: inputs.Workload, mode: str, causal: bool = True, chunks: int = 0,
                         curves: int = 0, bits: int = 10) -> float:
    """Bytes of one selection launch (all (b,h)) of a variant, counted as the kernels read
    them: 8 B per tree entry probed or windowed, the query code, idx out."""
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


VARIANTS = [  # name, zeta_select_opts fields (topk: a wider selection of the same workload)
    ("exact_k128", dict(mode=0, causal=True, topk=128)),
    ("exact_k256", dict(mode=0, causal=True, topk=256)),
    ("exact_noncausal", dict(mode=0, causal=False)),
    ("exact_12bit", dict(mode=0, causal=True, bits=12)),
    ("chunked_4", dict(mode=1, chunks=4)),
    ("chunked_8", dict(mode=1, chunks=8)),
    ("chunked_16", dict(mode=1, chunks=16)),
    ("chunked_32", dict(mode=1, chunks=32)),
    ("curves_3", dict(mode=2, curves=3)),
    ("curves_6", dict(mode=2, curves=6)),
]


def materialised_levels(w: inputs.Workload) -> int:
    """L_m = ceil(log2 N) - floor(log2 2k): tree levels the selection reads."""
    return max(0, int(np.ceil(np.log2(w.N))) - int(np.floor(np.log2(2 * w.topk))))


def algorithmic_bytes(w: inputs.Workload) -> dict:
    """Algorithmic bytes per launch of each stage, per query-head as the method's byte model
    fixes them (every gathered row counted as read; m = min(k, i+1) selected keys):
        encode   32 (q and k rows in, codes out)
        sort     4 + 8 L_m (codes in, one 8-byte entry per materialised level)
        select   4 + 4k + per run of size s: 2k * 8 + 4 log2(s) if s > 2k, else 4 s
        gather   4m + 12 + 12m + m dV|v| + dV|v|
        pass 1   m (16 + dV|v| + 8) + 12 + dV|v| + 12
        transp.  12k + 8
        pass 3   m (24 + dV|v|) + dV|v| + 24
    The processing-order builds and the dgamma reduction are not in that model; they are
    counted as the kernels move them (codes in, order out; one float per query)."""
    BH, N, k = w.B * w.H, w.N, w.topk
    vb = 2 if w.v_dtype == inputs.BF16 else 4
    row = w.dv * vb
    m = valid_slots(w).astype(np.float64)
    i1 = np.arange(1, N + 1, dtype=np.int64)
    runs = np.zeros(N, dtype=np.float64)
    for l in range(int(np.log2(N)) + 1):
        s = 1 << l
        has = ((i1 >> l) & 1).astype(np.float64)
        runs += has * ((2 * k * 8 + 4 * l) if s > 2 * k else 4 * s)
    b = {}
    b["encode_order"] = BH * N * (32 + 12)  # encode, then the query order (codes, placed, out)
    b["tree"] = BH * N * (4 + 8 * materialised_levels(w))
    b["select"] = BH * float((4 + 4 * k + runs).sum())
    b["order"] = 0  # built with the encodes on this path
    b["gather"] = BH * float((4 * m + 12 + 12 * m + m * row + row).sum())
    b["bwd_order"] = BH * N * (32 + 2 * 12)
    b["bwd_query"] = BH * float((m * (16 + row + 8) + 12 + row + 12).sum())
    b["bwd_transpose"] = BH * N * (12 * k + 8)
    b["bwd_key"] = BH * float((m * (24 + row) + row + 24).sum())
    b["bwd_dgamma"] = BH * N * 4.0
    return b


def compulsory_bytes(w: inputs.Workload, stored_levels: int) -> dict:
    """Bytes each stage must move through HBM at least: every distinct input byte it reads
    once and every output byte once (rows that many queries gather count once).  The trees
    are counted once written (tree) and once read (select); the transpose writes and reads
    its 8-byte records once and writes the 4-byte slot list and the segment bounds."""
    BH, N, k = w.B * w.H, w.N, w.topk
    vb = 2 if w.v_dtype == inputs.BF16 else 4
    row = w.dv * vb
    P = float(valid_slots(w).sum())  # pairs per (b,h)
    tree = 2 * 8 * stored_levels
    b = {}
    b["encode_order"] = BH * N * (24 + 8 + 4 + 4)
    b["tree"] = BH * N * (4 + tree)
    b["select"] = BH * (N * (4 + 4 + tree + 4 * k + 4))
    b["order"] = 0
    b["gather"] = BH * (N * (4 * k + 12 + 12 + row + row + 4))
    b["bwd_order"] = BH * N * (24 + 8 + 8 + 8)
    b["bwd_query"] = BH * (N * (4 * k + 12 + 12 + row + row + 8 * k + 12 + 4 + 4))
    b["bwd_transpose"] = BH * (N * 4 * k + P * (8 + 8 + 4) + N * 8)
    b["bwd_key"] = BH * (P * (4 + 8) + N * (12 + 12 + row + row + 12 + 8 + 4))
    b["bwd_dgamma"] = BH * N * 4.0
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


PROFILED = "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-variants --no-configs"
COPY = "python3 bench.py --copy-calibration"
# one counter group per run (rocprofv3 collects one pass per run)
COUNTER_CMDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o fetch -- " + PROFILED,
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o write -- " + PROFILED,
    "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d {d}/l2 -o l2 -- " + PROFILED,
    "rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_BUBBLE_sum --output-format csv "
    "-d {d}/ea -o ea -- " + PROFILED,
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_fetch -o copy_fetch -- " + COPY,
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_write -o copy_write -- " + COPY,
    "rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_BUBBLE_sum --output-format csv "
    "-d {d}/copy_ea -o copy_ea -- " + COPY,
    "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_WAVES SQ_WAVE_CYCLES "
    "SQ_BUSY_CYCLES --output-format csv -d {d}/lds -o lds -- " + PROFILED,
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
             "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-variants --no-configs"
             "{wl}")
CEILING_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o tr -- "
               "python3 bench.py --gather-ceiling")


def _maybe_means(path: str, counter: str) -> dict:
    return counter_means(path, counter) if os.path.isdir(path) else {}


def counters_summary(d: str, workload: str) -> None:
    """Bytes each kernel moves beyond L2 (FETCH_SIZE, WRITE_SIZE; each scaled by what the same
    counter reads for a plain 1 GiB device copy), the raw read requests beyond L2 by size,
    and the L2 hit rate (TCC_HIT, TCC_MISS); writes profiles/<stage>_<workload>_counters.json
    (keyed to the kernel source's sha256) and profiles/counters_<workload>.md."""
    copy_bytes = float(1 << 30)
    cf = counter_means(os.path.join(d, "copy_fetch"), "FETCH_SIZE")
    cw = counter_means(os.path.join(d, "copy_write"), "WRITE_SIZE")
    copy_name = next(k for k in cf if "copyBuffer" in k or "copy" in k.lower())
    fscale = copy_bytes / (cf[copy_name] * 1024.0)
    wscale = copy_bytes / (cw[copy_name] * 1024.0)
    fetch = counter_means(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = counter_means(os.path.join(d, "write"), "WRITE_SIZE")
    hit = _maybe_means(os.path.join(d, "l2"), "TCC_HIT_sum")
    miss = _maybe_means(os.path.join(d, "l2"), "TCC_MISS_sum")
    ea = {c: _maybe_means(os.path.join(d, "ea"), c)
          for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum")}
    cea = {c: _maybe_means(os.path.join(d, "copy_ea"), c)
           for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum")}
    cmds = [c.format(d=d) for c in COUNTER_CMDS]
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    lines = [f"# Memory traffic per launch, {workload} (rocprofv3 counters)", "",
             "Commands (each counter group its own run, from the repository root):", ""]
    lines += [f"    {c}" for c in cmds] + [f"    python3 bench.py --counters-summary {d}", ""]
    lines += [f"Copy calibration: a 1 GiB device copy reads {cf[copy_name]:.0f} KiB (FETCH_SIZE) and "
              f"writes {cw[copy_name]:.0f} KiB (WRITE_SIZE): scale {fscale:.3f} and {wscale:.3f}."]
    if cea["TCC_EA0_RDREQ_sum"].get(copy_name):
        creq = cea["TCC_EA0_RDREQ_sum"][copy_name]
        lines += [f"The copy makes {creq:.0f} read requests beyond L2 ({copy_bytes / creq:.1f} bytes "
                  f"each; {cea['TCC_EA0_RDREQ_32B_sum'].get(copy_name, 0):.0f} of 32 bytes, "
                  f"TCC_BUBBLE {cea['TCC_BUBBLE_sum'].get(copy_name, 0):.0f}).  The kernels' "
                  "request sizes are in the table: where their 32-byte share is as small as the "
                  "copy's, every request moves a whole 128-byte line and the copy's scale holds "
                  "for them too."]
    lines += ["", "FETCH_SIZE and WRITE_SIZE count traffic between L2 and the data fabric, which "
              "includes hits in the 256 MB Infinity Cache: an upper bound of the HBM bytes.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | beyond-L2 MB per launch (scaled) | "
              "read requests | of them 32 B | L2 hit rate |",
              "|---|---|---|---|---|---|---|"]

    def hbm(k):
        return fetch[k] * 1024 * fscale + write.get(k, 0.0) * 1024 * wscale

    def l2rate(k):
        h, mm = hit.get(k), miss.get(k)
        return h / (h + mm) if h is not None and mm is not None and h + mm > 0 else None

    for kname in sorted(fetch, key=lambda n: -fetch[n]):
        if not kname.startswith("zeta_"):
            continue
        req = ea["TCC_EA0_RDREQ_sum"].get(kname)
        r32 = ea["TCC_EA0_RDREQ_32B_sum"].get(kname)
        rate = l2rate(kname)
        lines.append(f"| {kname} | {fetch[kname]:.0f} | {write.get(kname, 0.0):.0f} | "
                     f"{hbm(kname) / 1e6:.1f} | {'-' if req is None else f'{req:.0f}'} | "
                     f"{'-' if r32 is None else f'{r32:.0f}'} | "
                     f"{'-' if rate is None else f'{rate:.1%}'} |")
    for stage, kname in SINGLE_KERNEL.items():
        if kname not in fetch:
            continue
        src = os.path.join(ROOT, "order_retrieval_amd", "csrc", KERNEL_SOURCE[stage])
        rec = {"kernel": kname, "workload": workload,
               "fetch_kib": fetch[kname], "write_kib": write.get(kname, 0.0),
               "fetch_scale": fscale, "write_scale": wscale,
               "hbm_bytes_per_launch": int(hbm(kname)),
               "l2_hit_rate": l2rate(kname),
               "source": KERNEL_SOURCE[stage],
               "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
               "commands": cmds}
        with open(os.path.join(prof, f"{stage}_{workload}_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
    tr = os.path.join(os.path.dirname(os.path.abspath(d)), "trace")
    kt = trace_kernels(tr) if os.path.isdir(tr) else {}
    if kt:
        lines += ["", f"Achieved rate beyond L2: the bytes above over the average kernel duration "
                  f"of the kernel trace in {tr} (the same bench command, its own run):", "",
                  "| kernel | beyond-L2 MB per launch | average us | GB/s | of 8 TB/s |",
                  "|---|---|---|---|---|"]
        for kname in sorted(fetch, key=lambda n: -fetch[n]):
            if not kname.startswith("zeta_") or kname not in kt:
                continue
            gbs = hbm(kname) / (kt[kname]["us"] * 1e-6) / 1e9
            lines.append(f"| {kname} | {hbm(kname) / 1e6:.1f} | {kt[kname]['us']:.1f} | {gbs:.0f} | "
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


def ceiling_summary(d: str) -> None:
    """profiles/gather_ceiling.md: the row-gather ceiling that bench.py --gather-ceiling
    printed (HIP events) next to the kernel trace of the same run."""
    stats = glob.glob(os.path.join(d, "*kernel_stats.csv"))
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    line = None
    log = os.path.join(d, "run.log")
    if os.path.exists(log):
        for ln in open(log):
            if ln.startswith("{"):
                line = json.loads(ln)
    durs = []  # probe dispatches in launch order: 3 warm-up then the timed ones, per table
    for f in glob.glob(os.path.join(d, "*kernel_trace.csv")):
        for r in csv.DictReader(open(f)):
            if kernel_base(r["Kernel_Name"]) == "zeta_probe_row_gather_kernel":
                durs.append((int(r["Start_Timestamp"]),
                             (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3))
    durs = [u for _, u in sorted(durs)]
    lines = ["# Row-gather ceiling (zeta_probe_row_gather)", "",
             "What bounds the gather and both backward passes: groups of 16 lanes each read 32 "
             "rows of 256 bytes drawn uniformly from a table, 16 bytes per lane, eight rows' "
             "loads in flight together (the access shape of those kernels, without their other "
             f"work); {CEILING_GROUPS} groups per launch, "
             f"{CEILING_GROUPS * CEILING_ROWS * CEILING_ROW_BYTES / 1e9:.2f} GB read per launch.  "
             "A 2 MiB table sits in every XCD's 4 MB L2; 16 MiB (one head's bf16 values at "
             "N = 65536, dV = 128) in the Infinity Cache; 1 GiB comes from HBM.", "",
             "Command (from the repository root; stdout to run.log in the same folder):", "",
             f"    {CEILING_CMD.format(d=d)}", f"    python3 bench.py --ceiling-summary {d}", ""]
    if line is not None:
        lines += ["| table | launches timed | GB/s (HIP events) | us per launch (HIP events) | "
                  "us per launch (kernel trace, same launches) |", "|---|---|---|---|---|"]
        at = 0
        for name, r in line["gather_ceiling"].items():
            n = r["launches"]
            timed = durs[at + 3: at + 3 + n]
            at += 3 + n
            tr_us = f"{sum(timed) / len(timed):.1f}" if len(timed) == n else "-"
            lines.append(f"| {name} | {n} | {r['GBs']:.0f} | {r['us']:.1f} | {tr_us} |")
    with open(os.path.join(ROOT, "profiles", "gather_ceiling.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def trace_summary(d: str, workload: str) -> None:
    """Per-kernel durations from a rocprofv3 --kernel-trace --stats run, next to the bench line
    the same run printed (its stage_ms come from HIP events on the launch stream)."""
    wl = "" if workload == "long_fwd_bwd" else f" --workload {workload}"
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
             f"    {TRACE_CMD.format(d=d, wl=wl)}",
             f"    python3 bench.py --trace-summary {d}{wl}", "",
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
    for name, f in VARIANTS:
        KK = f.get("topk", K)  # a wider selection of the same workload
        shape = Z.make_shape(w.B, w.H, N, w.dv, KK,
                             Z.ZETA_BF16 if v.dtype == torch.bfloat16 else Z.ZETA_F32)
        o = Z.select_opts(f.get("mode", 0), causal=f.get("causal", True), bits=f.get("bits", 10),
                          chunks=f.get("chunks", 0), curves=f.get("curves", 0))
        ws_f = Z.workspace(shape, Z.ZETA_WS_FWD, q.device, o)
        ws_b = Z.workspace(shape, Z.ZETA_WS_BWD, q.device, o)
        idx = torch.empty((w.B, w.H, N, KK), dtype=torch.int32, device=q.device)
        for _ in range(2):
            Z.zeta_fwd_ex(q, k, v, gamma, KK, o, ws=ws_f, out=out, idx=idx)
            Z.zeta_bwd_ex(q, k, v, gamma, idx, dout, o, ws=ws_b, grads=grads)
        ev = [(hip.create(6), hip.create(6)) for _ in range(steps)]
        torch.cuda.synchronize()
        for ef, eb in ev:
            lib.zeta_set_stage_events(ef, 6)
            Z.zeta_fwd_ex(q, k, v, gamma, KK, o, ws=ws_f, out=out, idx=idx)
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
        wk = inputs.Workload(**{**w.__dict__, "topk": KK})
        sb = variant_select_bytes(wk, mode, f.get("causal", True), f.get("chunks", 0),
                                  f.get("curves", 0), f.get("bits", 10))
        sel_rows = idx.reshape(BH, N, KK)[:, rows]
        r = {"select_stages_ms": round(sel, 4), "select_kernel_ms": round(sel_k, 4),
             "fwd_ms": round(fwd, 4), "fwd_bwd_ms": round(fwd + bwd, 4),
             "select_algorithmic_GBs": round(sb / ((sel if mode == "curves" else sel_k) * 1e-3)
                                             / 1e9, 1)}
        if KK == K:
            r["recall_vs_exact_causal"] = round(_recall(sel_rows, exact_rows, torch), 4)
            r["recall_vs_euclidean"] = round(_recall(sel_rows, eu_causal if f.get("causal", True)
                                                     else eu_all, torch), 4)
        else:  # the exact top-KK against the Euclidean top-KK of the same queries
            r["topk"] = KK
            r["recall_vs_euclidean"] = round(
                _recall(sel_rows, _euclid_topk(q, k, rows, KK, True, torch), torch), 4)
        if mode == "curves":  # stage 3 spans the later curves and the merge
            r["note"] = "select_kernel_ms covers curves 2..P and the merge; GB/s over all stages"
        res[name] = r
        del ws_f, ws_b
    return res


# ----------------------------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
            "kind": "oracle", "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": (f"{count} uniformly drawn query rows of the same workload (select + forward "
                       f"+ backward contributions, {t:.1f} s), scaled by {total}/{count}; "
                       f"selection and forward use all threads, backward runs on one")}


# ----------------------------------------------------------------------------- GPU runs
def measure_ceiling(Z, torch, launches: int = 10) -> dict:
    """Rate of scattered 16-lane 256-byte row gathers (zeta_probe_row_gather) per table size,
    timed with events on the launch stream."""
    res = {}
    sink = torch.empty(CEILING_GROUPS, dtype=torch.int32, device="cuda")
    nbytes = CEILING_GROUPS * CEILING_ROWS * CEILING_ROW_BYTES
    for name, size in CEILING_TABLES:
        table = torch.randint(0, 255, (size,), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            Z.zeta_probe_row_gather(table, CEILING_ROW_BYTES, CEILING_GROUPS, CEILING_ROWS, 1, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for t in range(launches):
            Z.zeta_probe_row_gather(table, CEILING_ROW_BYTES, CEILING_GROUPS, CEILING_ROWS, 2 + t,
                                    sink)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / launches
        res[name] = {"GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "us": round(us, 2),
                     "launches": launches, "bytes": nbytes}
        del table
    return res


class Run:
    """One workload resident on the device, with its workspaces and outputs."""

    def __init__(self, w: inputs.Workload, Z, torch):
        self.w, self.Z, self.torch = w, Z, torch
        x = inputs.make_inputs(w)
        self.sha = inputs.digest(x)
        dev = torch.device("cuda", 0)
        bf = w.v_dtype == inputs.BF16

        def to_dev(a, as_bf16=False):
            if as_bf16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        self.q, self.k, self.gamma = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["gamma"])
        self.v, self.dout = to_dev(x["v"], bf), to_dev(x["dout"], bf)
        self.shape = Z.make_shape(w.B, w.H, w.N, w.dv, w.topk, Z.ZETA_BF16 if bf else Z.ZETA_F32)
        self.ws_f = Z.workspace(self.shape, Z.ZETA_WS_FWD, dev)
        self.ws_b = Z.workspace(self.shape, Z.ZETA_WS_BWD, dev)
        self.out = torch.empty_like(self.v)
        self.idx = torch.empty((w.B, w.H, w.N, w.topk), dtype=torch.int32, device=dev)
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v),
                      torch.empty((w.H,), dtype=torch.float32, device=dev))
        self.x = x

    def fwd(self):
        self.Z.zeta_fwd(self.q, self.k, self.v, self.gamma, self.w.topk, ws=self.ws_f,
                        out=self.out, idx=self.idx)

    def bwd(self):
        self.Z.zeta_bwd(self.q, self.k, self.v, self.gamma, self.idx, self.dout, ws=self.ws_b,
                        grads=self.grads)


def time_run(r: Run, lib, hip, steps: int, warmup: int) -> dict:
    """The fwd+bwd step and the forward alone (events around `steps` back-to-back calls, the
    library's stage events off), then the stage times from HIP events the library records
    between its stages on a second pass of `steps` calls (each recorded event also leaves a
    gap of a few microseconds between two kernels, so that pass's total is reported apart as
    `instrumented_step_ms`)."""
    torch = r.torch
    for _ in range(warmup):
        r.fwd()
        r.bwd()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        r.fwd()
        r.bwd()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / steps

    ev = [(hip.create(len(FWD_STAGES) + 1), hip.create(len(BWD_STAGES) + 1))
          for _ in range(steps)]
    torch.cuda.synchronize()
    i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    i0.record()
    for evf, evb in ev:
        lib.zeta_set_stage_events(evf, len(evf))
        r.fwd()
        lib.zeta_set_stage_events(evb, len(evb))
        r.bwd()
        lib.zeta_set_stage_events(None, 0)
    i1.record()
    torch.cuda.synchronize()
    stages = {n: [] for n in FWD_STAGES + BWD_STAGES}
    for evf, evb in ev:
        for s_, n in enumerate(FWD_STAGES):
            stages[n].append(hip.elapsed_ms(evf[s_], evf[s_ + 1]))
        for s_, n in enumerate(BWD_STAGES):
            stages[n].append(hip.elapsed_ms(evb[s_], evb[s_ + 1]))
        hip.destroy(evf)
        hip.destroy(evb)
    stage_ms = {n: float(np.mean(t)) for n, t in stages.items()}
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record()
    for _ in range(steps):
        r.fwd()
    f1.record()
    torch.cuda.synchronize()
    return {"step_ms": step_ms, "fwd_only_ms": f0.elapsed_time(f1) / steps, "stage_ms": stage_ms,
            "instrumented_step_ms": i0.elapsed_time(i1) / steps, "wall_s": wall}


def stored_levels(w: inputs.Workload) -> int:
    """Tree levels the forward workspace stores (causal selection): from log2(2K) (K = k padded
    to a power of two; shorter runs are read from the codes) to the top level floor(log2(N-1))
    (a run of N keys, the last query's when N is a power of two, is read as two runs of the
    level below; kept when that level is below log2(2K)), and from the tile stage's top level
    (12) when that is lower and merge passes build the rest from it."""
    K = 1
    while K < w.topk:
        K *= 2
    first = int(np.log2(2 * K))
    L = (w.N - 1).bit_length() if w.N >= 2 else 1
    if L - 1 < first:
        L = w.N.bit_length()
    top_tile = min(L - 1, 12)
    base = top_tile if (top_tile + 1 < L and first > top_tile) else first
    return max(0, L - base)


def summarise(r: Run, t: dict) -> dict:
    """Per-workload figures: times, queries/s, bytes and fractions."""
    w = r.w
    alg = algorithmic_bytes(w)
    comp = compulsory_bytes(w, stored_levels(w))
    sm = t["stage_ms"]
    fwd_stage_ms = sum(sm[n] for n in FWD_STAGES)
    fwd_alg = sum(alg[n] for n in FWD_STAGES)
    fwd_comp = sum(comp[n] for n in FWD_STAGES)
    step_alg = sum(alg.values())
    step_comp = sum(comp.values())
    rows = w.B * w.H * w.N
    kern = {}
    for n in FWD_STAGES + BWD_STAGES:
        if sm[n] <= 0 or alg[n] == 0:
            continue
        kern[n] = {"ms": round(sm[n], 4), "algorithmic_bytes": int(alg[n]),
                   "compulsory_bytes": int(comp[n]),
                   "effective_GBs": round(alg[n] / (sm[n] * 1e-3) / 1e9, 1),
                   "hbm_frac_compulsory": round(comp[n] / (sm[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return {
        "shape": f"B{w.B} H{w.H} N{w.N} dK3 dV{w.dv} k{w.topk} v/dO {w.v_dtype} {w.dist}",
        "fwd_ms": round(t["fwd_only_ms"], 4),
        "fwd_bwd_ms": round(t["step_ms"], 4),
        "instrumented_step_ms": round(t["instrumented_step_ms"], 4),
        "queries_per_s_fwd": round(rows / (t["fwd_only_ms"] * 1e-3), 1),
        "queries_per_s_fwd_bwd": round(rows / (t["step_ms"] * 1e-3), 1),
        "fwd_algorithmic_bytes": int(fwd_alg),
        "fwd_effective_GBs": round(fwd_alg / (fwd_stage_ms * 1e-3) / 1e9, 1),
        "fwd_compulsory_bytes": int(fwd_comp),
        "fwd_hbm_frac": round(fwd_comp / (fwd_stage_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_effective_GBs": round(step_alg / (t["step_ms"] * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_comp / (t["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stage_ms": {n: round(v, 4) for n, v in sm.items()},
        "kernels": kern,
        "input_sha256": r.sha,
    }


def roofline(summary: dict, ceiling: dict) -> dict:
    """The dominant single-kernel stage against what bounds it.  The row kernels gather rows
    that are mostly L2 hits, so their ceiling is the measured rate of such gathers (an
    L2-resident table); the selection is bounded by VALU issue and reported against HBM."""
    stages = {n: summary["kernels"][n] for n in SINGLE_KERNEL if n in summary["kernels"]}
    dom = max(stages, key=lambda n: stages[n]["ms"])
    st = stages[dom]
    ms = st["ms"]
    traffic = stored_traffic(dom)
    peak = ceiling["l2_2MiB"]["GBs"]
    hbm = {"compulsory_bytes": st["compulsory_bytes"],
           "achieved": round(st["compulsory_bytes"] / (ms * 1e-3) / 1e9, 1),
           "peak": HBM_PEAK_GBS, "frac": st["hbm_frac_compulsory"]}
    dram = None if traffic is None else {
        "bytes": traffic, "GBs": round(traffic / (ms * 1e-3) / 1e9, 1),
        "frac": round(traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return {"bound": "vmem" if dom in ROW_KERNELS else "hbm", "kernel": SINGLE_KERNEL[dom],
            "stage": dom, "ms": ms, "achieved": st["effective_GBs"],
            "peak": peak if dom in ROW_KERNELS else HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(st["effective_GBs"] / (peak if dom in ROW_KERNELS else HBM_PEAK_GBS), 4),
            "traffic": traffic,
            "peak_kind": ("measured in this run: scattered 16-lane 256-byte row gathers from an "
                          "L2-resident table (zeta_probe_row_gather), the access these kernels make"
                          if dom in ROW_KERNELS else "MI355X HBM3E, published"),
            "achieved_kind": "the stage's algorithmic bytes (every gathered row counted as read) "
                             "over its HIP-event duration",
            "hbm": hbm, "dram": dram}


def memory_footprint(w: inputs.Workload, Z, torch) -> dict:
    """Device memory of one forward and one forward+backward through the autograd wrapper
    (inputs, outputs, index tensor, gradients and the per-call workspaces), from a clean
    allocator state."""
    bf = w.v_dtype == inputs.BF16
    x = inputs.make_inputs(w)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def to_dev(a, as_bf16=False):
        if as_bf16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(a).to("cuda")

    q, k, g = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["gamma"])
    v, dout = to_dev(x["v"], bf), to_dev(x["dout"], bf)
    with torch.no_grad():
        out, idx = Z.zeta_fwd(q, k, v, g, w.topk)
    torch.cuda.synchronize()
    peak_fwd = torch.cuda.max_memory_allocated() - base
    del out, idx
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    qr, kr, vr, gr = (t.clone().requires_grad_() for t in (q, k, v, g))
    out, idx = Z.zeta_attention(qr, kr, vr, gr, w.topk)
    out.backward(dout)
    torch.cuda.synchronize()
    peak_step = torch.cuda.max_memory_allocated() - base
    shape = Z.make_shape(w.B, w.H, w.N, w.dv, w.topk, Z.ZETA_BF16 if bf else Z.ZETA_F32)
    res = {"fwd_workspace_MB": round(Z.zeta_workspace_bytes(shape, Z.ZETA_WS_FWD) / 1e6, 1),
           "bwd_workspace_MB": round(Z.zeta_workspace_bytes(shape, Z.ZETA_WS_BWD) / 1e6, 1),
           "peak_allocated_MB_fwd": round(peak_fwd / 1e6, 1),
           "peak_allocated_MB_fwd_bwd": round(peak_step / 1e6, 1),
           "note": ("torch.cuda.max_memory_allocated over one zeta_fwd, and over one forward + "
                    "backward through zeta_attention (the fwd+bwd figure also holds a copy of "
                    "q, k, v, gamma made to request gradients); pages' context: 17348.2 MB for "
                    "ZETA and 10516.1 MB for FlashAttention at 65536 tokens, shapes unstated")}
    del qr, kr, vr, gr, out, idx, q, k, g, v, dout
    torch.cuda.empty_cache()
    return res


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other synthetic configurations and the memory footprint")
    ap.add_argument("--variant-steps", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device-to-device copies (counter calibration)")
    ap.add_argument("--gather-ceiling", action="store_true",
                    help="only measure the row-gather ceiling (zeta_probe_row_gather)")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="write profiles/*_counters.json from rocprofv3 --pmc outputs under DIR")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 kernel-trace run")
    ap.add_argument("--ceiling-summary", metavar="DIR",
                    help="write profiles/gather_ceiling.md from a traced --gather-ceiling run")
    args = ap.parse_args()
    if args.counters_summary:
        counters_summary(args.counters_summary, args.workload)
        return 0
    if args.trace_summary:
        trace_summary(args.trace_summary, args.workload)
        return 0
    if args.ceiling_summary:
        ceiling_summary(args.ceiling_summary)
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

    if args.gather_ceiling:
        print(json.dumps({"gather_ceiling": measure_ceiling(Z, torch)}), flush=True)
        return 0

    lib = Z.load_library()
    hip = HipEvents(Z.hip_runtimes_mapped()[0])
    w = inputs.CONFIGS[args.workload]
    w = inputs.Workload(**{**w.__dict__, "backward": True})
    r = Run(w, Z, torch)
    torch.cuda.synchronize()
    t = time_run(r, lib, hip, args.steps, args.warmup)
    main_sum = summarise(r, t)
    ceiling = measure_ceiling(Z, torch)
    roof = roofline(main_sum, ceiling)
    result = {
        "metric": METRIC,
        "value": round(t["step_ms"], 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["step_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} H{w.H} N{w.N} dK3 dV{w.dv} k{w.topk}, "
                               f"v/dO {w.v_dtype}, forward+backward",
                   "B": w.B, "H": w.H, "N": w.N, "d_K": 3, "d_V": w.dv, "topk": w.topk,
                   "v_dtype": w.v_dtype, "seed": w.seed},
        **{k_: main_sum[k_] for k_ in ("fwd_ms", "fwd_bwd_ms", "queries_per_s_fwd",
                                       "queries_per_s_fwd_bwd", "fwd_algorithmic_bytes",
                                       "fwd_effective_GBs", "fwd_compulsory_bytes", "fwd_hbm_frac",
                                       "step_effective_GBs", "step_hbm_frac", "stage_ms",
                                       "kernels")},
        "roofline": roof,
        "gather_ceiling": ceiling,
        "wall_s_timed": round(t["wall_s"], 3),
        "pages_context": PAGES_CONTEXT,
        "input_sha256": r.sha,
    }
    idx_main = r.idx
    if not args.no_variants:
        result["variants"] = measure_variants(w, r.q, r.k, r.v, r.gamma, r.dout, idx_main, hip, lib,
                                              Z, torch, args.variant_steps)
    x_main = r.x
    del r
    torch.cuda.empty_cache()
    if not args.no_configs:
        configs = {}
        for name, cw in inputs.CONFIGS.items():
            if name in ("long_fwd", "long_fwd_bwd") and w.name in ("long_fwd", "long_fwd_bwd"):
                s_ = {k_: v_ for k_, v_ in main_sum.items() if k_ != "kernels"}
            else:
                rr = Run(inputs.Workload(**{**cw.__dict__, "backward": True}), Z, torch)
                s_ = summarise(rr, time_run(rr, lib, hip, args.steps, args.warmup))
                s_.pop("kernels")
                del rr
                torch.cuda.empty_cache()
            if name == "long_fwd":  # the forward of the 65536-token workload (same inputs)
                s_ = {k_: v_ for k_, v_ in s_.items() if not k_.startswith(("fwd_bwd", "step_"))
                      and k_ != "queries_per_s_fwd_bwd"}
            configs[name] = s_
        result["configs"] = configs
        result["memory"] = memory_footprint(w, Z, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x_main, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
