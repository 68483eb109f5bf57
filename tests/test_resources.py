"""Scratch gate over the compiled kernels (no GPU): the compiler's resource report of the last
build (memory_bound_amd/build.py keeps it in _build/resource_usage.txt) must show no scratch
memory -- no spilled registers -- in any kernel, except the allow-list below, none of whose
entries any workload launches.  A kernel that starts spilling after a change fails here instead
of only slowing down.
"""
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

SCRATCH = "ScratchSize [bytes/lane]"

# Mangled-name patterns allowed to use scratch, with the reason.  Nothing in the benchmark or
# any workload launches these.
ALLOWED = {
    r"^_ZN4fuse19cumsum_scale_kernelILNS_2DTE[012]ELb0ELi32ELi8ELi1EE":
        "per-element cumsum path at 32 elements per lane and 8 waves per row: only rows of 8193 to "
        "16384 elements that are not a whole number of 16-byte words take it",
}

# Demangled names of the instantiations the workloads launch (the benchmark's rows).
WORKLOAD_KERNELS = [
    "add_layernorm_kernel<(fuse::DT)1, true, 2, 4, true, 4>",      # Add+LN fp16 [2048,4096]
    "add_layernorm_kernel<(fuse::DT)1, true, 2, 4, true, 2>",      # Add+LN fp16 [16384,4096]
    "ew_kernel<(fuse::DT)1, true, 2, fuse::OpBiasGeluRes>",       # BiasAdd+GELU+Residual
    "softmax_rows_kernel<(fuse::DT)1, true, 2, 2, true>",          # softmax [65536,2048]
    "cumsum_scale_kernel<(fuse::DT)1, true, 2, 4, 2>",             # cumsum + scale
    "swiglu_persist_kernel<4, 0>",                                 # SwiGLU 2048x8960x1536
    "swiglu_persist_kernel<4, 3>",                                 # GEMM + bias + ReLU
]


@pytest.fixture(scope="module")
def table():
    from memory_bound_amd import build
    path = os.path.join(ROOT, "_build", "resource_usage.txt")
    if not os.path.exists(path) or not os.path.exists(build.LIB):
        build.build()
    return build.resource_table(path)


def _demangle(names):
    cxxfilt = shutil.which("c++filt")
    if cxxfilt is None:
        pytest.skip("no c++filt")
    out = subprocess.run([cxxfilt], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
    return dict(zip(names, out))


def test_no_scratch_outside_the_allow_list(table):
    assert len(table) > 100
    bad = [f"{k}: {v[SCRATCH]} B/lane, {v.get('VGPRs Spill', 0)} VGPRs spilled" for k, v in table.items()
           if v.get(SCRATCH, 0) > 0 and not any(re.search(p, k) for p in ALLOWED)]
    assert not bad, "\n".join(bad)


def test_workload_kernels_are_present_and_spill_free(table):
    dem = _demangle(list(table))
    for want in WORKLOAD_KERNELS:
        hits = [k for k, d in dem.items() if want in d]
        assert hits, f"{want} not in the build"
        for k in hits:
            assert table[k].get(SCRATCH, 0) == 0 and table[k].get("VGPRs Spill", 0) == 0, (want, table[k])


def test_allow_list_entries_are_not_workload_kernels(table):
    dem = _demangle(list(table))
    for k, d in dem.items():
        if any(re.search(p, k) for p in ALLOWED):
            assert not any(w in d for w in WORKLOAD_KERNELS), d
