"""Scratch gate over the compiled kernels (no GPU): the compiler's resource report of the last
build (memory_bound_amd/build.py keeps it in _build/resource_usage.txt) must show no scratch
memory -- no spilled registers -- in any kernel of the library.  A kernel that starts spilling
after a change fails here instead of only slowing down.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SCRATCH = "ScratchSize [bytes/lane]"

# Demangled names of the instantiations the workloads launch (the benchmark's rows).
WORKLOAD_KERNELS = [
    "add_layernorm_kernel<(fuse::DT)1, true, 2, 4, true, 4>",      # Add+LN fp16 [2048,4096]
    "add_layernorm_kernel<(fuse::DT)1, true, 2, 4, true, 2>",      # Add+LN fp16 [16384,4096]
    "add_layernorm_ex_kernel<(fuse::DT)1, true, 1, 8, true, 4>",   # LN+ReLU, sum and statistics
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


def test_no_kernel_uses_scratch(table):
    assert len(table) > 100
    bad = [f"{k}: {v[SCRATCH]} B/lane, {v.get('VGPRs Spill', 0)} VGPRs spilled" for k, v in table.items()
           if v.get(SCRATCH, 0) > 0 or v.get("VGPRs Spill", 0) > 0]
    assert not bad, "\n".join(bad)


def test_workload_kernels_are_present_and_spill_free(table):
    dem = _demangle(list(table))
    for want in WORKLOAD_KERNELS:
        hits = [k for k, d in dem.items() if want in d]
        assert hits, f"{want} not in the build"
        for k in hits:
            assert table[k].get(SCRATCH, 0) == 0 and table[k].get("VGPRs Spill", 0) == 0, (want, table[k])
