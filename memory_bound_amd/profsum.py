"""Summaries of rocprofv3 results (the rocpd SQLite database it writes) per kernel and grid size.

    python -m memory_bound_amd.profsum trace  <results.db>   # dispatch durations
    python -m memory_bound_amd.profsum pmc    <results.db>   # hardware counter values
    python -m memory_bound_amd.profsum dispatches <results.db> <kernel>
        # one kernel, per dispatch: duration (a --kernel-trace run) and every counter collected
    python -m memory_bound_amd.profsum clock  <results.db> <kernel> <flop>
        # per dispatch of a --kernel-trace run with SQ_CYCLES and SQ_VALU_MFMA_BUSY_CYCLES: shader
        # clock, matrix-core busy fraction, achieved TFLOP/s for `flop` per dispatch, bf16 peak at
        # that clock (MI355X: 32 shader engines, 1024 SIMDs, 1024 bf16 flop per SIMD per cycle)
    python -m memory_bound_amd.profsum hbm    <fetch.db> <write.db>
        # bytes moved per dispatch from a FETCH_SIZE run and a WRITE_SIZE run of the same
        # program, each counter scaled by what it reads for the plain copy of 24 MiB in that run
    python -m memory_bound_amd.profsum sweep  <results.db>
        # a `bench.py --sweep` run: Add+LayerNorm and copy kernel medians per size, and the line
        # t = t0 + bytes / bw fitted to each
    python -m memory_bound_amd.profsum headline <results.db> <n_cold>
        # the headline kernel in a trace of the default benchmark: its first n_cold (cold)
        # dispatches as `key: value` lines that bench.py reads back, with the source hash
    python -m memory_bound_amd.profsum split  <results.db> <kernel> <grid> <n>
        # one kernel at one grid size: its first n dispatches and the rest, apart (a benchmark
        # that times the same kernel first on rotating cold buffers, then on one hot buffer set)
    python -m memory_bound_amd.profsum headline-counters <fetch.db> <write.db>
        # a `bench.py --counters` FETCH_SIZE run and WRITE_SIZE run: the raw counter means of the
        # calibration copy, the headline kernel and the unfused chains, the scale factors, and the
        # `key: value` lines bench.py reads back (HBM bytes per dispatch, unfused over fused)
    python -m memory_bound_amd.profsum rows   <fetch.db> <write.db>
        # a `bench.py --counters-rows` FETCH_SIZE run and WRITE_SIZE run: per row of the path
        # other than the headline, the bytes its kernels moved (as `hbm` scales them) against the
        # row's algorithmic bytes, fused and unfused
    python -m memory_bound_amd.profsum splits <bench.json>
        # the JSON line of `bench.py --split-sweep` as a table: per shape, the split-K plan's
        # choice and time, the fastest forced split count, how far off the plan is, and every
        # forced split count's time (this mode reads the benchmark's output, not a database)

rocprofv3's own --stats table groups dispatches by kernel name only; the same kernel
instantiation runs at several shapes here (the [2048,4096] and [16384,4096] Add+LayerNorm share
one), so the tables below also split by grid size.  Durations are in microseconds; counter values
are what rocprofv3 reports per dispatch (FETCH_SIZE and WRITE_SIZE in KiB).
"""
from __future__ import annotations

import json
import sqlite3
import statistics
import sys
from collections import defaultdict


def short_name(name: str) -> str:
    i = name.rfind(">(")
    n = name[: i + 1] if i > 0 else name.split("(")[0]
    return n.replace("void ", "").replace("fuse::", "").replace("(anonymous namespace)::", "").replace("(DT)", "")


def _stats(d: list[float]) -> dict:
    q = statistics.quantiles(d, n=10, method="inclusive") if len(d) > 1 else [d[0]] * 9
    return {"calls": len(d), "mean_us": statistics.mean(d), "median_us": statistics.median(d),
            "p10_us": q[0], "p90_us": q[8], "min_us": min(d), "max_us": max(d)}


def trace(db_path: str) -> list[dict]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x, workgroup_x, duration from kernels order by start").fetchall()
    g = defaultdict(list)
    for name, gx, wx, dur in rows:
        g[(short_name(name), gx, wx)].append(dur / 1e3)
    return [{"kernel": n, "grid": gx, "wg": wx, **_stats(d)} for (n, gx, wx), d in g.items()]


def split(db_path: str, kernel: str, grid: int, first: int) -> tuple[dict, dict | None]:
    """Durations of `kernel` (its short name) at `grid`, in dispatch order: the first `first`
    dispatches and the rest."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x, duration from kernels order by start").fetchall()
    d = [dur / 1e3 for name, gx, dur in rows if gx == grid and short_name(name) == kernel]
    if len(d) < first or first < 1:
        raise SystemExit(f"{kernel} at grid {grid}: {len(d)} dispatches, fewer than {first}")
    return _stats(d[:first]), (_stats(d[first:]) if len(d) > first else None)


def dispatches(db_path: str, kernel: str) -> list[dict]:
    """Per dispatch of `kernel` (its short name), in order: duration in us and counter values."""
    db = sqlite3.connect(db_path)
    dur = {d: t / 1e3 for n, d, t in db.execute("select name, dispatch_id, duration from kernels")
           if short_name(n) == kernel}
    out = defaultdict(dict)
    for n, d, c, v in db.execute("select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        if short_name(n) == kernel:
            out[d][c] = v
    return [{"dispatch": d, "us": dur.get(d), **out[d]} for d in sorted(set(dur) | set(out))]


SHADER_ENGINES, SIMDS, BF16_FLOP_PER_SIMD_CYCLE = 32, 1024, 1024


def clock(db_path: str, kernel: str, flop: float) -> list[dict]:
    """Per dispatch: duration, clock (SQ_CYCLES per engine over the duration), MFMA busy fraction
    (busy cycles per SIMD over cycles per engine), achieved TFLOP/s and the peak at that clock."""
    out = []
    for r in dispatches(db_path, kernel):
        eng = r["SQ_CYCLES"] / SHADER_ENGINES
        mhz = eng / r["us"]
        out.append({"us": r["us"], "mhz": mhz, "mfma_busy": r["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / eng,
                    "tflops": flop / (r["us"] * 1e-6) / 1e12,
                    "peak_tflops": SIMDS * BF16_FLOP_PER_SIMD_CYCLE * mhz * 1e6 / 1e12})
    return out


COPY_KERNEL, COPY_BYTES = "copy16_kernel<4>", 24 << 20  # the calibration copy: 24 MiB read, 24 MiB written


def hbm(fetch_db: str, write_db: str) -> tuple[float, float, list[dict]]:
    """Per kernel and grid: mean FETCH_SIZE and WRITE_SIZE (KiB) and the bytes they stand for.
    Each counter is scaled by the bytes the calibration copy in the same run moves over what the
    counter reads for it."""
    mean = {}
    for db, cname in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        for r in pmc(db):
            if r["counter"] == cname:
                mean[(r["kernel"], r["grid"], cname)] = r["mean"]
    copy = [k for k in mean if k[0] == COPY_KERNEL and k[1] == COPY_BYTES // 64]
    if len(copy) != 2:
        raise SystemExit("the runs hold no 24 MiB calibration copy")
    fs = COPY_BYTES / 1024 / mean[(COPY_KERNEL, COPY_BYTES // 64, "FETCH_SIZE")]
    ws = COPY_BYTES / 1024 / mean[(COPY_KERNEL, COPY_BYTES // 64, "WRITE_SIZE")]
    out = []
    for (k, g) in sorted({(k, g) for k, g, _ in mean}, key=lambda t: (t[0], t[1])):
        f, w = mean.get((k, g, "FETCH_SIZE")), mean.get((k, g, "WRITE_SIZE"))
        if f is None or w is None:
            continue
        out.append({"kernel": k, "grid": g, "fetch_kib": f, "write_kib": w,
                    "bytes": f * 1024 * fs + w * 1024 * ws})
    return fs, ws, out


def pmc(db_path: str) -> list[dict]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, grid_size, workgroup_size, counter_name, value "
                      "from counters_collection order by dispatch_id").fetchall()
    g = defaultdict(list)
    for name, grid, wg, cname, val in rows:
        g[(short_name(name), grid, wg, cname)].append(val)
    out = []
    for (n, grid, wg, cname), v in g.items():
        out.append({"kernel": n, "grid": grid, "wg": wg, "counter": cname, "calls": len(v),
                    "mean": statistics.mean(v), "median": statistics.median(v), "min": min(v), "max": max(v)})
    return out


HEADLINE_SOURCES = ["fuse_common.hpp", "row_plan.hpp", "row_plan.hip", "row_kernels.hpp", "row_launch.hpp"]
HEADLINE_KERNEL, HEADLINE_GRID = "add_layernorm_kernel<1, true, 2, 4, true, 4>", 131072


def source_hash(files=HEADLINE_SOURCES) -> str:
    """sha256 prefix of the kernel sources a profile was taken with (memory_bound_amd/csrc)."""
    import hashlib
    import os
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_profile(path: str) -> dict | None:
    """The `key: value` lines of a committed profile summary, or None when the file is missing or
    the kernel sources changed since it was taken (its kernel_source_sha256)."""
    import os
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0] if v.strip() else ""
    return kv if kv.get("kernel_source_sha256") == source_hash() else None


def headline(db_path: str, cold: int) -> dict:
    """The headline kernel's first `cold` dispatches in a trace of the default benchmark (the
    eager, warm-up and timed launches, each on a buffer set not touched for 1 GiB)."""
    head, rest = split(db_path, HEADLINE_KERNEL, HEADLINE_GRID, cold)
    return {"cold": head, "hot": rest}


SWEEP_ROWS, SWEEP_HIDDEN = (512, 1024, 2048, 4096, 8192, 16384, 32768), 4096


def sweep(db_path: str, skip: int = 3) -> dict:
    """Kernel durations of a `bench.py --sweep` run: for each size in turn, its Add+LayerNorm
    dispatches, then its copy dispatches (the first `skip` of each, eager warm-up launches,
    dropped).  Groups are runs of consecutive dispatches of one kernel at one grid.  Each size's
    median and a least-squares line t = t0 + bytes / bw per kernel (fp16 at H = 4096: 3 row
    tensors plus gamma and beta for Add+LayerNorm, the same 3 tensors' bytes for the copy)."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x, duration from kernels order by start").fetchall()
    groups = []
    for name, gx, dur in rows:
        n = short_name(name)
        if not (n.startswith("add_layernorm_kernel") or n.startswith("copy16_kernel")):
            continue
        if not groups or groups[-1][0] != (n, gx):
            groups.append(((n, gx), []))
        groups[-1][1].append(dur / 1e3)
    if len(groups) != 2 * len(SWEEP_ROWS):
        raise SystemExit(f"expected {2 * len(SWEEP_ROWS)} groups (Add+LN, copy per size), found {len(groups)}")
    sizes = []
    for i, r in enumerate(SWEEP_ROWS):
        (ln_k, ln_g), ln_d = groups[2 * i]
        (cp_k, cp_g), cp_d = groups[2 * i + 1]
        t = 3 * r * SWEEP_HIDDEN * 2
        sizes.append({"rows": r, "bytes": t + 2 * SWEEP_HIDDEN * 2, "copy_bytes": t, "ln_kernel": ln_k,
                      "ln_grid": ln_g, "ln": _stats(ln_d[skip:]), "copy": _stats(cp_d[skip:])})
    fits = {}
    for key, bkey in (("ln", "bytes"), ("copy", "copy_bytes")):
        xs = [s[bkey] for s in sizes]
        ys = [s[key]["median_us"] for s in sizes]
        mx, my = statistics.mean(xs), statistics.mean(ys)
        b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
        fits[key] = {"t0_us": my - b * mx, "bw_gbps": 1e-3 / b}
    return {"sizes": sizes, "fits": fits}


# The rows of `bench.py --counters-rows`: label, workload (its algorithmic bytes come from
# roofline.workload_work), fused or not, and the (kernel, grid) dispatches that make it up.
ROW_TRAFFIC = (
    ("LN+ReLU, sum, mean/var fp16 [2048,4096]", ("add_layernorm_ex", (2048, 4096), "f16"), True,
     (("add_layernorm_ex_kernel<1, true, 1, 8, true, 4>", 262144),)),
    ("cumsum+scale fp16 [2048,4096]", "cumsum_f16_2048x4096", True, (("cumsum_scale_kernel<1, true, 2, 4, 2>", 262144),)),
    ("  unfused: scan + scale", "cumsum_f16_2048x4096", False,
     (("cumsum_scale_kernel<1, true, 2, 4, 2>", 262144), ("ew_kernel<1, true, 2, OpScale>", 524288))),
    ("softmax fp16 [65536,2048]", "softmax_f16_65536x2048", True, (("softmax_rows_kernel<1, true, 2, 2, true>", 8388608),)),
    ("  unfused: max, exp+sum, divide", "softmax_f16_65536x2048", False,
     (("softmax_rowmax_kernel<1, true>", 4194304), ("softmax_expsum_kernel<1, true>", 4194304),
      ("softmax_divide_kernel<1, true>", 4194304))),
    ("SwiGLU bf16 2048x8960x1536", "swiglu_bf16_2048x8960x1536", True, (("swiglu_persist_kernel<4, 0>", 65536),)),
    ("  unfused: products + SiLU*", "swiglu_bf16_2048x8960x1536", False,
     (("swiglu_persist_kernel<4, 1>", 65536), ("ew_kernel<2, true, 4, OpSiluMul>", 573440))),
    ("GEMM+bias+ReLU bf16 2048x8960x1536", "gemm_relu_bf16_2048x8960x1536", True, (("swiglu_persist_kernel<4, 3>", 65536),)),
    ("  unfused: GEMM, bias, ReLU", "gemm_relu_bf16_2048x8960x1536", False,
     (("swiglu_persist_kernel<4, 2>", 65536), ("ew_kernel<2, true, 4, OpBiasAdd>", 573440),
      ("ew_kernel<2, true, 4, OpRelu>", 573440))),
)


def row_traffic(fetch_db: str, write_db: str) -> str:
    """The ROW_TRAFFIC table from a FETCH_SIZE run and a WRITE_SIZE run, as text."""
    from memory_bound_amd import roofline, synth
    fs, ws, rows = hbm(fetch_db, write_db)
    by = {(r["kernel"], r["grid"]): r for r in rows}
    c = by[(COPY_KERNEL, COPY_BYTES // 64)]
    out = [f"# Calibration in the same runs: a copy of exactly 24 MiB reads FETCH_SIZE {c['fetch_kib']:.2f} KiB "
           f"and WRITE_SIZE", f"# {c['write_kib']:.2f} KiB, so counter KiB x {fs:.5f} (fetch) and x {ws:.5f} "
           f"(write) are bytes moved.",
           f"{'row':41s} {'measured_bytes':>14s} {'algorithmic':>13s} {'ratio':>7s}   kernels (fetch KiB / write KiB)"]
    for label, work, fused, kernels in ROW_TRAFFIC:
        op, shape, dtype = work if isinstance(work, tuple) else (synth.WORKLOADS[work].op, synth.WORKLOADS[work].shape,
                                                                 synth.WORKLOADS[work].dtype)
        alg = roofline.workload_work(op, shape, dtype, fused)["bytes"]
        m = round(sum(by[k]["bytes"] for k in kernels))
        out.append(f"{label:41s} {m:14d} {alg:13d} {m / alg:7.3f}   "
                   + "; ".join(f"{k[0]} {by[k]['fetch_kib']:.0f}/{by[k]['write_kib']:.0f}" for k in kernels))
    return "\n".join(out)


# The kernels of `bench.py --counters`: label and (kernel, grid).
COUNTER_KERNELS = (
    ("copy 24 MiB", (COPY_KERNEL, COPY_BYTES // 64)),
    ("fused Add+LayerNorm", (HEADLINE_KERNEL, HEADLINE_GRID)),
    ("unfused: add kernel", ("ew_kernel<1, true, 2, OpAdd>", 524288)),
    ("unfused: LayerNorm kernel", ("add_layernorm_kernel<1, true, 2, 4, false, 4>", 131072)),
    ("fused BiasAdd+GELU+Residual", ("ew_kernel<1, true, 2, OpBiasGeluRes>", 524288)),
    ("unfused: bias kernel", ("ew_kernel<1, true, 2, OpBiasAdd>", 524288)),
    ("unfused: GELU kernel", ("ew_kernel<1, true, 2, OpGelu>", 524288)),
)


def headline_counters(fetch_db: str, write_db: str) -> str:
    """The headline counter summary (raw means, scales, the key lines bench.py reads) as text."""
    from memory_bound_amd import roofline
    fs, ws, rows = hbm(fetch_db, write_db)
    by = {(r["kernel"], r["grid"]): r for r in rows}
    b = {label: by[kg]["bytes"] for label, kg in COUNTER_KERNELS}
    ln_alg = roofline.workload_work("add_layernorm", (2048, 4096), "f16", True)["bytes"]
    ln_unf_alg = roofline.workload_work("add_layernorm", (2048, 4096), "f16", False)["bytes"]
    ge_alg = roofline.workload_work("bias_gelu_residual", (2048, 4096), "f16", True)["bytes"]
    ge_unf_alg = roofline.workload_work("bias_gelu_residual", (2048, 4096), "f16", False)["bytes"]
    fused, unf = b["fused Add+LayerNorm"], b["unfused: add kernel"] + b["unfused: LayerNorm kernel"]
    ge, ge_unf = (b["fused BiasAdd+GELU+Residual"],
                  b["unfused: bias kernel"] + b["unfused: GELU kernel"] + b["unfused: add kernel"])
    out = ["# Raw counter means per dispatch (KiB):"]
    for label, kg in COUNTER_KERNELS:
        r = by[kg]
        out.append(f"#   {label:30s} {kg[0]:44s} FETCH_SIZE {r['fetch_kib']:10.2f}  WRITE_SIZE {r['write_kib']:10.2f}")
    out += ["#   (the unfused GELU chain ends with the same add kernel as the unfused Add+LayerNorm)", "#",
            f"fetch_scale: {fs:.5f}", f"write_scale: {ws:.5f}", "#",
            "# Scaled HBM bytes per dispatch (fetch * fetch_scale + write * write_scale, in bytes):",
            f"kernel: {HEADLINE_KERNEL} grid {HEADLINE_GRID}",
            f"kernel_source_sha256: {source_hash()}",
            f"hbm_bytes_per_dispatch: {round(fused)}", f"algorithmic_bytes_per_dispatch: {ln_alg}",
            f"traffic_over_algorithmic: {fused / ln_alg:.4f}",
            f"unfused_chain_hbm_bytes: {round(unf)}", f"unfused_chain_algorithmic_bytes: {ln_unf_alg}",
            f"unfused_over_fused_traffic: {unf / fused:.4f}",
            f"gelu_fused_hbm_bytes: {round(ge)}   (algorithmic {ge_alg})",
            f"gelu_unfused_chain_hbm_bytes: {round(ge_unf)}   (algorithmic {ge_unf_alg}; ratio {ge_unf / ge:.3f})"]
    return "\n".join(out)


def split_table(path: str) -> str:
    """The `bench.py --split-sweep` JSON line (the last line of `path` starting with '{') as text."""
    line = [l for l in open(path).read().splitlines() if l.startswith("{")][-1]
    rows = json.loads(line)["split_sweep"]
    counts = sorted({int(k) for r in rows for k in r["forced"]})
    out = [f"{'op':6s} {'M x N x K':>16s} {'plan':>5s} {'plan_us':>8s} {'best':>5s} {'best_us':>8s} {'off':>6s}  "
           + " ".join(f"{'s=' + str(c):>7s}" for c in counts)]
    for r in rows:
        m, n, k = r["shape"]
        best, best_us = r["best_forced"]
        cells = " ".join(f"{r['forced'][str(c)]:7.2f}" if str(c) in r["forced"] else f"{'-':>7s}" for c in counts)
        out.append(f"{r['op']:6s} {f'{m}x{n}x{k}':>16s} {r['plan_splits']:5d} {r['plan_us']:8.2f} {best:5d} "
                   f"{best_us:8.2f} {(r['plan_us'] / best_us - 1) * 100:5.1f}%  {cells}")
    return "\n".join(out)


def main(argv):
    mode, path = argv[1], argv[2]
    if mode == "splits":
        print(split_table(path))
        return
    if mode == "rows":
        print(row_traffic(path, argv[3]))
        return
    if mode == "headline-counters":
        print(headline_counters(path, argv[3]))
        return
    if mode == "trace":
        print(f"{'kernel':64s} {'grid':>9s} {'wg':>4s} {'calls':>5s} {'mean_us':>9s} {'median_us':>9s} "
              f"{'p10_us':>8s} {'p90_us':>8s} {'min_us':>8s} {'max_us':>8s}")
        for r in trace(path):
            print(f"{r['kernel'][:64]:64s} {r['grid']:9d} {r['wg']:4d} {r['calls']:5d} {r['mean_us']:9.3f} "
                  f"{r['median_us']:9.3f} {r['p10_us']:8.3f} {r['p90_us']:8.3f} {r['min_us']:8.3f} "
                  f"{r['max_us']:8.3f}")
    elif mode == "pmc":
        print(f"{'kernel':64s} {'grid':>9s} {'counter':>11s} {'calls':>5s} {'mean':>12s} {'median':>12s}")
        for r in pmc(path):
            print(f"{r['kernel'][:64]:64s} {r['grid']:9d} {r['counter']:>11s} {r['calls']:5d} {r['mean']:12.2f} "
                  f"{r['median']:12.2f}")
    elif mode == "dispatches":
        rows = dispatches(path, argv[3])
        names = sorted({k for r in rows for k in r} - {"dispatch", "us"})
        print(f"{'dispatch':>9s} {'us':>9s} " + " ".join(f"{n:>26s}" for n in names))
        for r in rows:
            us = f"{r['us']:9.3f}" if r["us"] is not None else f"{'-':>9s}"
            print(f"{r['dispatch']:9d} {us} " + " ".join(f"{r.get(n, float('nan')):26.0f}" for n in names))
    elif mode == "clock":
        rows = clock(path, argv[3], float(argv[4]))
        print("dispatch       us    MHz mfma_busy  TFLOP/s peak_at_clock")
        for i, r in enumerate(rows, 1):
            print(f"{i:8d} {r['us']:8.1f} {r['mhz']:6.0f} {r['mfma_busy']:9.3f} {r['tflops']:8.0f} "
                  f"{r['peak_tflops']:13.0f}")
        med = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
        print(f"  median {med['us']:8.1f} {med['mhz']:6.0f} {med['mfma_busy']:9.3f} {med['tflops']:8.0f} "
              f"{med['peak_tflops']:13.0f}")
    elif mode == "hbm":
        fs, ws, rows = hbm(path, argv[3])
        print(f"# fetch_scale {fs:.5f}  write_scale {ws:.5f}  (24 MiB copy in the same runs)")
        print(f"{'kernel':64s} {'grid':>9s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'bytes':>12s}")
        for r in rows:
            print(f"{r['kernel'][:64]:64s} {r['grid']:9d} {r['fetch_kib']:11.2f} {r['write_kib']:11.2f} "
                  f"{r['bytes']:12.0f}")
    elif mode == "sweep":
        r = sweep(path)
        print(f"{'rows':>6s} {'MB_moved':>9s} {'addln_med_us':>12s} {'p10':>7s} {'p90':>7s} {'frac':>6s} "
              f"{'copy_med_us':>11s} {'p10':>7s} {'p90':>7s} {'frac':>6s}  kernel")
        for z in r["sizes"]:
            ln, cp = z["ln"], z["copy"]
            print(f"{z['rows']:6d} {z['bytes'] / 1e6:9.2f} {ln['median_us']:12.3f} {ln['p10_us']:7.3f} "
                  f"{ln['p90_us']:7.3f} {z['bytes'] / (ln['median_us'] * 1e-6) / 8e12:6.3f} {cp['median_us']:11.3f} "
                  f"{cp['p10_us']:7.3f} {cp['p90_us']:7.3f} {z['copy_bytes'] / (cp['median_us'] * 1e-6) / 8e12:6.3f}  "
                  f"{z['ln_kernel']} grid {z['ln_grid']}")
        for k, f in r["fits"].items():
            name = "Add+LayerNorm" if k == "ln" else "copy"
            print(f"fit {name:13s} t = {f['t0_us']:.3f} us + bytes / {f['bw_gbps']:.1f} GB/s "
                  f"({f['bw_gbps'] / 8000:.3f} of 8 TB/s)")
    elif mode == "headline":
        r = headline(path, int(argv[3]))
        c = r["cold"]
        print(f"kernel: {HEADLINE_KERNEL} grid {HEADLINE_GRID}")
        print(f"kernel_source_sha256: {source_hash()}")
        print(f"cold_dispatches: {c['calls']}")
        for k in ("mean", "median", "p10", "p90", "min", "max"):
            print(f"cold_{k}_us: {c[k + '_us']:.3f}")
        if r["hot"]:
            print(f"hot_dispatches: {r['hot']['calls']}")
            print(f"hot_mean_us: {r['hot']['mean_us']:.3f}")
    elif mode == "split":
        head, rest = split(path, argv[3], int(argv[4]), int(argv[5]))
        for label, r in (("first", head), ("rest", rest)):
            if r:
                print(f"{label:5s} calls {r['calls']:5d} mean {r['mean_us']:.3f} median {r['median_us']:.3f} "
                      f"p10 {r['p10_us']:.3f} p90 {r['p90_us']:.3f} min {r['min_us']:.3f} max {r['max_us']:.3f} us")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
