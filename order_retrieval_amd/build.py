"""Build ``libzeta.so`` (hand-written HIP for gfx950) in-tree.

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 only, then the objects are
linked against the HIP runtime that PyTorch loads (``torch/lib/libamdhip64.so``), so the
library and torch share one runtime, one device context and the same streams.

Usage: ``python -m order_retrieval_amd.build`` (or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import glob
import importlib.util
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libzeta.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    "-c", "-fPIC", "-O3", "-std=c++17", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is not importable; it provides the HIP runtime to link against")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {d}")
    return d


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link libzeta.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *HIP_FLAGS, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tdir = torch_lib_dir()
    tmp = LIB + ".tmp"
    link = ["g++", "-shared", "-o", tmp, *objs, f"-L{tdir}", "-lamdhip64",
            f"-Wl,-rpath,{tdir}", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif "warning" in text and "packed-fp32-ops" not in text:
            sys.stderr.write(text)
    procs.clear()
    if failed:
        for src, text in failed:
            sys.stderr.write(f"--- {src}\n{text}\n")
        raise RuntimeError(f"hipcc failed for {[os.path.basename(s) for s, _ in failed]}")


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
