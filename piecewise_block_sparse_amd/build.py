"""Build libpisa.so (gfx950) in-tree with hipcc.

    python -m piecewise_block_sparse_amd.build          # or build() from Python

Each HIP source is compiled to an object with hipcc for gfx950 and the objects
are linked into piecewise_block_sparse_amd/libpisa.so; the measurement probe
(csrc/probe_rate.hip, include/pisa_probe.h) becomes libpisa_probe.so.  The
compile always runs (no up-to-date check), so a call after editing a source
rebuilds it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpisa.so")
PROBE_LIB = os.path.join(PKG, "libpisa_probe.so")
SOURCES = ["api.hip", "attn_bf16.hip", "attn_f32.hip", "stats.hip", "route.hip"]
PROBE_SOURCES = ["probe_rate.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        objs = [o for (o, _), src in zip(results, SOURCES + PROBE_SOURCES) if src in srcs]
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
