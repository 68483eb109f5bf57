"""Host-side logic without a GPU: seeded inputs, comparison rules, roofline arithmetic."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from memory_bound_amd import roofline, synth
from oracle import tolerance


# ---- seeded inputs -----------------------------------------------------------------------------

def test_inputs_are_deterministic_and_seed_dependent():
    a = synth.add_layernorm_inputs(8, 96, "f16", 1003)
    b = synth.add_layernorm_inputs(8, 96, "f16", 1003)
    c = synth.add_layernorm_inputs(8, 96, "f16", 1004)
    for k in ("x", "residual", "gamma", "beta"):
        assert torch.equal(a[k], b[k])
        assert a[k].dtype == torch.float16
    assert not torch.equal(a["x"], c["x"])


def test_inputs_distributions():
    d = synth.add_layernorm_inputs(256, 4096, "f32", 1)
    x = d["x"].double()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
    assert d["gamma"].min() >= 0.5 and d["gamma"].max() <= 1.5
    assert abs(d["beta"].double().std().item() - 0.1) < 0.01
    s = synth.softmax_inputs(64, 2048, "f16", 2)
    assert abs(s["x"].double().std().item() - math.sqrt(128)) < 0.2
    assert s["scale"] == 1 / math.sqrt(128)
    w = synth.swiglu_inputs(64, 512, 1536, "bf16", 3)
    assert w["a"].dtype == torch.bfloat16 and w["b1"].shape == (1536, 512)
    assert abs(w["b1"].double().std().item() - 1 / math.sqrt(1536)) < 1e-3
    g = synth.bias_gelu_residual_inputs(64, 4096, "f16", 4)
    assert abs(g["bias"].double().std().item() - 0.02) < 0.003


def test_workload_table():
    w = synth.WORKLOADS
    assert w["addln_f16_2048x4096"].shape == (2048, 4096)
    assert w["addln_f16_16384x4096"].shape == (8 * 2048, 4096)
    assert w["softmax_f16_65536x2048"].shape == (32 * 2048, 2048)
    assert w["swiglu_bf16_2048x8960x1536"].shape == (2048, 8960, 1536)
    assert w["cumsum_f16_2048x4096"].shape == (2048, 4096)
    assert len({x.seed for x in w.values()}) == len(w)
    c = w["cumsum_f16_2048x4096"].inputs()
    assert c["x"].dtype == torch.float16 and c["scale"] == 1 / 64
    assert abs(c["x"].double().std().item() - 1) < 0.01


# ---- comparison rules --------------------------------------------------------------------------

def test_ulp16():
    v = np.array([1.0, 1.5, 8.0, 9.0, 2.0 ** -14, 2.0 ** -20, 0.0, -4.0])
    np.testing.assert_array_equal(tolerance.ulp16(v), [2.0 ** -10, 2.0 ** -10, 2.0 ** -7, 2.0 ** -7,
                                                       2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -8])


def test_compare_rules():
    ref = np.array([0.5, 10.0, -3.0])
    assert tolerance.compare(ref + [1.9e-3, 7e-3, -1.9e-3], ref, "f16")["ok"]
    assert not tolerance.compare(ref + [2.1e-3, 0, 0], ref, "f16")["ok"]
    assert not tolerance.compare(ref + [0, 8e-3, 0], ref, "f16")["ok"]
    # bf16: relative with a 1e-2 floor
    assert tolerance.compare([1.009, 0.0, 5e-3 + 9e-5], [1.0, 0.0, 5e-3], "bf16")["ok"]
    assert not tolerance.compare([1.011], [1.0], "bf16")["ok"]
    assert not tolerance.compare([2e-4], [0.0], "bf16")["ok"]
    assert tolerance.compare([1.0 + 9e-6], [1.0], "f32")["ok"]
    assert not tolerance.compare([1.0 + 2e-5], [1.0], "f32")["ok"]
    # NaN must match NaN
    assert not tolerance.compare([np.nan], [1.0], "f32")["ok"]
    assert not tolerance.compare([1.0], [np.nan], "f32")["ok"]
    assert tolerance.compare([np.nan], [np.nan], "f32")["ok"]


def test_perfect_fp16_rounding_meets_the_rule():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(100000) * 4
    y = ref.astype(np.float16).astype(np.float64)
    assert tolerance.compare(y, ref, "f16")["ok"]


# ---- roofline arithmetic against the page's own traffic figures ----------------------------------

def test_traffic_matches_page_three_section_one():
    mib = {k: int(v) for k, v in read_golden("traffic_page3.txt")}
    rows, hidden = 1 * 2048, 4096
    tensor = rows * hidden * 2
    assert tensor == mib["tensor_mib"] << 20
    fused = roofline.add_layernorm_bytes(rows, hidden, "f16", fused=True)
    unfused = roofline.add_layernorm_bytes(rows, hidden, "f16", fused=False)
    assert fused["tensor_bytes"] == mib["fused_total_mib"] << 20
    assert unfused["tensor_bytes"] == mib["unfused_total_mib"] << 20
    assert (mib["unfused_add_mib"] + mib["unfused_layernorm_mib"]) == mib["unfused_total_mib"]
    # with gamma and beta: 3 * 16 MiB + 2 * 8 KiB
    assert fused["bytes"] == 50_348_032


def test_other_algorithmic_work():
    assert roofline.bias_gelu_residual_bytes(2048, 4096, "f16")["bytes"] == 50_339_840
    assert roofline.softmax_rows_bytes(65536, 2048, "f16")["bytes"] == 536_870_912
    assert roofline.swiglu_flops(2048, 8960, 1536) == 112_742_891_520
    assert roofline.add_layernorm_bytes(64, 768, "f32")["bytes"] == 595_968
    assert roofline.add_layernorm_bytes(16384, 4096, "f16")["bytes"] == 402_669_568
    # LayerNorm variants: one more tensor (the pre-norm sum) and 8 bytes of statistics per row
    assert roofline.add_layernorm_ex_bytes(2048, 4096, "f16")["bytes"] == 50_348_032 + 16_777_216 + 16_384
    # cumsum + scale: read x, write y; unfused adds the stored prefix sums and their reload
    assert roofline.cumsum_scale_rows_bytes(2048, 4096, "f16")["bytes"] == 33_554_432
    assert roofline.cumsum_scale_rows_bytes(2048, 4096, "f16", fused=False)["bytes"] == 67_108_864
    assert roofline.gemm_flops(2048, 8960, 1536) == 56_371_445_760
    assert roofline.gemm_bias_act_bytes(2048, 8960, 1536, "bf16")["bytes"] == 2 * (2048 * 1536 + 1536 * 8960 + 8960 + 2048 * 8960)


def test_oracle_thread_count_round_trip():
    # the one-thread timing in the bench's CPU baseline sets and restores the OpenMP thread count;
    # the result must not depend on it
    import oracle

    n = oracle.threads()
    d = synth.add_layernorm_inputs(8, 256, "f16", seed=5)
    x, r, g, b = (oracle.f64(d[k]) for k in ("x", "residual", "gamma", "beta"))
    y_all = oracle.add_layernorm(x, r, g, b, 1e-5)
    oracle.set_threads(1)
    try:
        assert oracle.threads() == 1
        assert np.array_equal(oracle.add_layernorm(x, r, g, b, 1e-5), y_all)
    finally:
        oracle.set_threads(n)
    assert oracle.threads() == n


def test_bench_refuses_more_than_one_gpu():
    # the path is single-GPU: asking the benchmark for N > 1 GPUs ends with a message and a
    # non-zero status before anything touches a device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for n in ("2", "8"):
        p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", n], capture_output=True,
                           text=True, timeout=120)
        assert p.returncode == 2, p.stderr
        assert "one GPU only" in p.stderr and not p.stdout.strip()


def test_profile_summary_scales_counters_by_the_calibration_copy(tmp_path):
    # FETCH_SIZE and WRITE_SIZE of a kernel become bytes through the ratio the 24 MiB copy of the
    # same run gives: here the copy reads back half its bytes on FETCH_SIZE and all on WRITE_SIZE
    import sqlite3
    from memory_bound_amd import profsum
    dbs = []
    for cname, copy_kib, k_kib in (("FETCH_SIZE", 12288.0, 1000.0), ("WRITE_SIZE", 24576.0, 2000.0)):
        path = str(tmp_path / f"{cname}.db")
        db = sqlite3.connect(path)
        db.execute("create table counters_collection (dispatch_id, kernel_name, grid_size, workgroup_size, "
                   "counter_name, value)")
        rows = [(1, "void fuse::copy16_kernel<4>(uint4 const*, uint4*, unsigned long)", 393216, 256, cname, copy_kib),
                (2, "void fuse::k<1, true>(float const*)", 100, 256, cname, k_kib),
                (3, "void fuse::k<1, true>(float const*)", 100, 256, cname, k_kib + 2.0)]
        db.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
        db.commit()
        dbs.append(path)
    fs, ws, out = profsum.hbm(*dbs)
    assert fs == 2.0 and ws == 1.0
    k = [r for r in out if r["kernel"] == "k<1, true>"][0]
    assert k["fetch_kib"] == 1001.0 and k["write_kib"] == 2001.0
    assert k["bytes"] == 1001.0 * 1024 * 2 + 2001.0 * 1024
    c = [r for r in out if r["kernel"] == "copy16_kernel<4>"][0]
    assert c["bytes"] == 2 * (24 << 20)


def test_profile_row_traffic_table(tmp_path):
    # every kernel of the rows table reads 1000 KiB on FETCH_SIZE and 500 on WRITE_SIZE, with the
    # copy calibrating both counters at 1:1 bytes; a row's measured bytes are then 1500 KiB per
    # kernel, set against the row's algorithmic bytes
    import sqlite3
    from memory_bound_amd import profsum, roofline, synth
    kernels = sorted({k for _, _, _, ks in profsum.ROW_TRAFFIC for k in ks})
    dbs = []
    for cname, copy_kib, k_kib in (("FETCH_SIZE", 24576.0, 1000.0), ("WRITE_SIZE", 24576.0, 500.0)):
        path = str(tmp_path / f"{cname}.db")
        db = sqlite3.connect(path)
        db.execute("create table counters_collection (dispatch_id, kernel_name, grid_size, workgroup_size, "
                   "counter_name, value)")
        rows = [(1, "void fuse::copy16_kernel<4>(uint4 const*, uint4*, unsigned long)", 393216, 256, cname, copy_kib)]
        rows += [(i + 2, f"void fuse::{k}(int)", g, 256, cname, k_kib) for i, (k, g) in enumerate(kernels)]
        db.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
        db.commit()
        dbs.append(path)
    lines = profsum.row_traffic(*dbs).splitlines()
    body = {l[:41].strip(): l for l in lines[3:]}
    assert len(body) == len(profsum.ROW_TRAFFIC)
    softmax_unfused = body["unfused: max, exp+sum, divide"].split()
    alg = roofline.workload_work("softmax_rows", synth.WORKLOADS["softmax_f16_65536x2048"].shape, "f16", False)["bytes"]
    assert int(softmax_unfused[4]) == 3 * 1500 * 1024 and int(softmax_unfused[5]) == alg


def test_profile_headline_counter_lines(tmp_path):
    # the key lines bench.py reads back: with every kernel at 1000 KiB fetched and 500 written and
    # the copy calibrating both counters 1:1, the fused kernel moves 1500 KiB and the unfused
    # add -> LayerNorm pair twice that
    import sqlite3
    from memory_bound_amd import profsum
    dbs = []
    for cname, k_kib in (("FETCH_SIZE", 1000.0), ("WRITE_SIZE", 500.0)):
        path = str(tmp_path / f"h{cname}.db")
        db = sqlite3.connect(path)
        db.execute("create table counters_collection (dispatch_id, kernel_name, grid_size, workgroup_size, "
                   "counter_name, value)")
        rows = [(i, f"void fuse::{kg[0]}(int)", kg[1], 256, cname, 24576.0 if kg[0] == profsum.COPY_KERNEL else k_kib)
                for i, (_, kg) in enumerate(profsum.COUNTER_KERNELS)]
        db.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
        db.commit()
        dbs.append(path)
    text = profsum.headline_counters(*dbs)
    kv = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith("#"))
    assert int(kv["hbm_bytes_per_dispatch"]) == 1500 * 1024
    assert kv["unfused_over_fused_traffic"] == "2.0000"
    assert kv["kernel_source_sha256"] == profsum.source_hash()


def test_profile_summary_clock_and_matrix_core_busy(tmp_path):
    # one dispatch of 1 us with 2000 cycles per shader engine runs at 2000 MHz; busy cycles of
    # half the SIMD-cycles give a busy fraction of 0.5; 1 GFLOP in 1 us is 1000 TFLOP/s
    import sqlite3
    from memory_bound_amd import profsum
    path = str(tmp_path / "clk.db")
    db = sqlite3.connect(path)
    db.execute("create table kernels (name, dispatch_id, duration)")
    db.execute("create table counters_collection (kernel_name, dispatch_id, counter_name, value)")
    name = "void fuse::k<4, 0>(fuse::DualArgs)"
    db.execute("insert into kernels values (?, 7, 1000)", (name,))
    db.executemany("insert into counters_collection values (?, 7, ?, ?)",
                   [(name, "SQ_CYCLES", 32 * 2000.0), (name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000.0)])
    db.commit()
    (r,) = profsum.clock(path, "k<4, 0>", 1e9)
    assert r["us"] == 1.0 and r["mhz"] == 2000.0 and r["mfma_busy"] == 0.5
    assert abs(r["tflops"] - 1000.0) < 1e-9
    assert abs(r["peak_tflops"] - 1024 * 1024 * 2e9 / 1e12) < 1e-9


def test_profiles_name_kernels_the_library_still_has():
    # every kernel a committed profile summary names (outside torch's own) is a __global__
    # function of the library's sources, with as many template arguments as its template has
    # parameters, so that a renamed or re-templated kernel shows up as a stale summary
    import pathlib
    import re
    root = pathlib.Path(__file__).resolve().parent.parent
    src = "\n".join(p.read_text() for p in sorted((root / "memory_bound_amd" / "csrc").iterdir())
                    if p.suffix in (".hip", ".hpp", ".h"))
    arity = {}
    for m in re.finditer(r"(?:template\s*<([^>]*)>\s*)?__global__\s+void\s+(?:__launch_bounds__\([^)]*\)\s*)?"
                         r"(\w+_kernel)\s*\(", src):
        arity[m.group(2)] = len(m.group(1).split(",")) if m.group(1) else 0
    assert {"add_layernorm_kernel", "swiglu_persist_kernel", "copy16_kernel", "empty_kernel"} <= set(arity)
    named = 0
    for prof in sorted((root / "profiles").glob("*.txt")):
        for m in re.finditer(r"(?<![\w:])(\w+_kernel)(?!\w)(?:<([^<>\n]*)>)?", prof.read_text()):
            name, args = m.group(1), m.group(2)
            assert name in arity, f"{prof.name} names {name}, which the library no longer defines"
            if args is not None:
                assert len(args.split(",")) == arity[name], f"{prof.name}: {name}<{args}>"
            named += 1
    assert named > 50
