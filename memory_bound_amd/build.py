"""Build libfuse.so (all HIP sources under csrc/) for gfx950, in-tree.

Each translation unit is compiled by hipcc in parallel into _build/, then linked into
memory_bound_amd/libfuse.so.  The per-kernel register / LDS / spill report the compiler emits
(-Rpass-analysis=kernel-resource-usage) is kept in _build/resource_usage.txt.

Usage: python -m memory_bound_amd.build [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfuse.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++20", "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-Rpass-analysis=kernel-resource-usage",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr[-8000:]}")
    return obj, p.stderr


def resource_table(path: str | None = None) -> dict[str, dict[str, int]]:
    """Per kernel (mangled name): the compiler's resource figures from the report of the last
    build -- VGPRs, AGPRs, SGPRs, spilled VGPRs / SGPRs and scratch bytes per lane."""
    path = path or os.path.join(BUILD, "resource_usage.txt")
    table, cur = {}, None
    for line in open(path):
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            table[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+(?:\[bytes/lane\])?): (\d+)", line)
        if m and cur:
            table[cur][m.group(1).strip()] = int(m.group(2))
    return table


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    report = "\n".join(r for _, r in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(report)
    spills = [ln for ln in report.splitlines()
              if re.search(r"(SGPRs|VGPRs) Spill: [1-9]", ln) or re.search(r"ScratchSize \[bytes/lane\]: [1-9]", ln)]
    if spills and verbose:
        print("warning: register spills / scratch use:\n" + "\n".join(spills[:20]), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args()
    build(a.j, verbose=True)
