"""Benchmark of the fused row kernels on one MI355X.

Headline: fused ResidualAdd+LayerNorm, [B,S,H] = [1,2048,4096] fp16 (2048 rows x 4096), achieved
HBM GB/s.  One step = one launch over one [2048,4096] batch.  The K timed steps (and the W warmup
steps) are captured into one HIP graph each and replayed, so the host's per-call cost does not
leave the GPU idle between 7-microsecond kernels.  Every step uses a different buffer set; the
sets span more than 1 GiB so that no step finds its inputs in the 256 MB Infinity Cache left
there by an earlier step: the bytes come from HBM.

value = algorithmic bytes of K steps / wall time of the timed region (host clock, synchronized
on both sides).  roofline.achieved = algorithmic bytes of one launch / average launch duration,
from HIP events recorded on the launch stream around the timed replay.  The other rows of the
hot path (BiasAdd+GELU+Residual, row softmax, SwiGLU), their unfused baselines and a plain copy
are timed the same way and reported under "rows".  cpu_baseline times the CPU oracle on the
same workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]
Profiling and study modes (one JSON line each): --counters, --counters-rows, --dispatch WORKLOAD,
--sweep (size sweep of Add+LN and the copy), --split-sweep (split-K plan against forced splits).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "addln_f16_2048x4096"
ROTATE_BYTES = 1 << 30
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "add_layernorm_f16_2048x4096_counters.txt")
PROFILE_TRACE = os.path.join(ROOT, "profiles", "add_layernorm_f16_2048x4096_trace.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def read_counters():
    """HBM bytes per dispatch of the headline kernel and the unfused chain's bytes over them,
    from the committed counter summary; (None, None) when the kernel source changed since the
    counters were taken."""
    from memory_bound_amd import profsum
    kv = profsum.read_profile(PROFILE_COUNTERS)
    try:
        if not kv:
            return None, None
        return float(kv["hbm_bytes_per_dispatch"]), float(kv["unfused_over_fused_traffic"])
    except (KeyError, ValueError):
        return None, None


def read_trace(nbytes):
    """The headline kernel's cold dispatch durations from the committed kernel-trace summary of
    the default benchmark command (None when the kernel source changed since it was taken), with
    the bandwidth and fraction of peak they give."""
    from memory_bound_amd import profsum, roofline
    kv = profsum.read_profile(PROFILE_TRACE)
    if not kv:
        return None
    try:
        mean, med = float(kv["cold_mean_us"]), float(kv["cold_median_us"])
        out = {"definition": "rocprofv3 --kernel-trace duration of each cold dispatch of the headline kernel "
                             "in the default benchmark command (the eager, warm-up and timed launches); no "
                             "gap between kernels included",
               "source": os.path.relpath(PROFILE_TRACE, ROOT), "dispatches": int(kv["cold_dispatches"]),
               "mean_us": mean, "median_us": med, "p10_us": float(kv["cold_p10_us"]),
               "p90_us": float(kv["cold_p90_us"])}
    except (KeyError, ValueError):
        return None
    out["achieved"] = round(nbytes / (mean * 1e-6) / 1e9, 1)
    out["frac"] = round(out["achieved"] / roofline.HBM_PEAK_GBPS, 4)
    out["frac_median"] = round(nbytes / (med * 1e-6) / 1e9 / roofline.HBM_PEAK_GBPS, 4)
    return out


class Timed:
    """Captures `count` calls of launch(i) into a HIP graph on a private stream."""

    def __init__(self, torch, stream, launch, count):
        self.torch = torch
        self.stream = stream
        self.count = count
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            for i in range(count):
                launch(i)

    def run(self):
        """Replay once; returns (host seconds, event milliseconds)."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        self.graph.replay()
        e1.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, e0.elapsed_time(e1)


def single_dispatch_us(torch, stream, launch, n=10, spin_cycles=2_000_000):
    """Median duration of n dispatches timed one at a time, each after a device synchronisation.
    A spin kernel (about 1 ms) keeps the stream busy while the start event, the dispatch and the
    end event are enqueued, so the host's enqueue time is not part of what is timed."""
    ts = []
    for i in range(n):
        torch.cuda.synchronize()
        torch.cuda._sleep(spin_cycles)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return statistics.median(ts)


def rotation_sets(torch, tensors: dict, outputs: dict, min_bytes: int):
    """Copies of the input tensors (and fresh outputs) until the sets together span min_bytes."""
    per = sum(t.numel() * t.element_size() for t in tensors.values())
    per += sum(t.numel() * t.element_size() for t in outputs.values())
    n = max(2, math.ceil(min_bytes / per))
    sets = []
    for _ in range(n):
        s = {k: v.to("cuda").clone() for k, v in tensors.items()}
        s.update({k: torch.empty_like(v, device="cuda") for k, v in outputs.items()})
        sets.append(s)
    return sets


def time_launches(torch, stream, launch, n, warm=3):
    for i in range(warm):
        launch(i)
    torch.cuda.synchronize()
    t = Timed(torch, stream, launch, n)
    t.run()  # first replay warms the graph
    host_s, ev_ms = t.run()
    return host_s, ev_ms


def headline(torch, api, synth, roofline, steps, warmup):
    w = synth.WORKLOADS[HEADLINE]
    rows, hidden = w.shape
    d = w.inputs()
    gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
    sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"]}, ROTATE_BYTES)
    log(f"headline {HEADLINE}: {len(sets)} buffer sets")
    stream = torch.cuda.Stream()
    work = roofline.workload_work(w.op, w.shape, w.dtype)

    def launch(i):
        s = sets[i % len(sets)]
        api.fuse_add_layernorm(s["x"], s["r"], gamma, beta, d["eps"], y=s["y"])

    with torch.cuda.stream(stream):
        for i in range(3):
            launch(i)
        torch.cuda.synchronize()
        warm_graph = Timed(torch, stream, launch, max(1, warmup))
        timed_graph = Timed(torch, stream, lambda i: launch(i + warmup), steps)
        warm_graph.run()
        host_s, ev_ms = timed_graph.run()
        # the same kernel on one buffer set every launch: its 48 MiB stay in the 256 MB Infinity
        # Cache, so this is a cache figure, reported apart and never as HBM bandwidth
        hot = Timed(torch, stream, lambda i: launch(0), 200)
        hot.run()
        _, hot_ms = hot.run()
    avg_us = ev_ms * 1e3 / steps
    hot_us = hot_ms * 1e3 / 200
    return {
        "workload": w,
        "bytes": work["bytes"],
        "host_s": host_s,
        "avg_launch_us": avg_us,
        "value_gbps": work["bytes"] * steps / host_s / 1e9,
        "achieved_gbps": work["bytes"] / (avg_us * 1e-6) / 1e9,
        "sets": len(sets),
        "hot": {"avg_launch_us": round(hot_us, 3), "gbps": round(work["bytes"] / (hot_us * 1e-6) / 1e9, 1),
                "note": "same buffers every launch (Infinity Cache resident): not an HBM figure"},
    }


def other_rows(torch, api, synth, roofline, n_launch=40):
    """Each remaining row of the hot path, its unfused baseline, and the copy ceiling."""
    out = {}
    stream = torch.cuda.Stream()
    peak_bw = roofline.HBM_PEAK_GBPS

    def single_dispatch(us, work):
        # the matrix-core kernels: one dispatch at a time beside the back-to-back figure, whose
        # launches run with the clock at the board's power limit
        return {"single_dispatch_us": round(us, 3),
                "single_dispatch_tflops": round(work["flops"] / (us * 1e-6) / 1e12, 1),
                "note": "avg_launch_us: back-to-back launches (sustained); single_dispatch_us: median of "
                        "10 synchronised single dispatches"}

    def record(name, op, shape, dtype, fused, ev_ms, n, extra=None):
        work = roofline.workload_work(op, shape, dtype, fused)
        us = ev_ms * 1e3 / n
        r = {"avg_launch_us": round(us, 3), "algorithmic_bytes": work["bytes"]}
        if "flops" in work:
            tf = work["flops"] / (us * 1e-6) / 1e12
            r.update({"achieved_tflops": round(tf, 1), "peak_tflops": roofline.MFMA_PEAK_TFLOPS["bf16"],
                      "frac": round(tf / roofline.MFMA_PEAK_TFLOPS["bf16"], 4), "bound": "mfma"})
        else:
            gb = work["bytes"] / (us * 1e-6) / 1e9
            r.update({"achieved_gbps": round(gb, 1), "frac": round(gb / peak_bw, 4), "bound": "hbm"})
        if extra:
            r.update(extra)
        out[name] = r
        log(f"{name}: {us:.2f} us")

    def of_ceiling(name, ceiling):
        # the row against what the matrix cores sustain with no memory traffic at all
        r = out[name]
        r["frac_of_mfma_ceiling"] = {
            "single_dispatch": round(r["single_dispatch_tflops"] / ceiling["single_dispatch_tflops"], 4),
            "back_to_back": round(r["achieved_tflops"] / ceiling["achieved_tflops"], 4)}

    with torch.cuda.stream(stream):
        # headline shape, unfused
        w = synth.WORKLOADS[HEADLINE]
        d = w.inputs()
        gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
        sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"]}, ROTATE_BYTES)
        ws = api._workspace(api.FUSE_OP_ADD_LAYERNORM, *w.shape, 0, api.FUSE_F16, "cuda")

        def unf(i):
            s = sets[i % len(sets)]
            api.fuse_unfused_add_layernorm(s["x"], s["r"], gamma, beta, d["eps"], y=s["y"], workspace=ws)
        _, ev = time_launches(torch, stream, unf, n_launch)
        record("add_layernorm_unfused_f16_2048x4096", w.op, w.shape, w.dtype, False, ev, n_launch,
               {"note": "add kernel + LayerNorm kernel; bytes = the unfused chain's 5 tensor passes"})

        w = synth.WORKLOADS["addln_f16_16384x4096"]
        d = w.inputs()
        gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
        sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"]}, ROTATE_BYTES)
        del d

        def ln8(i):
            s = sets[i % len(sets)]
            api.fuse_add_layernorm(s["x"], s["r"], gamma, beta, 1e-5, y=s["y"])
        _, ev = time_launches(torch, stream, ln8, n_launch)
        record("add_layernorm_f16_16384x4096", w.op, w.shape, w.dtype, True, ev, n_launch)
        del sets

        w = synth.WORKLOADS["addln_f32_64x768"]
        d = w.inputs()
        g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
        y = torch.empty_like(g["x"])

        def ln_small(i):
            api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"], y=y)
        _, ev = time_launches(torch, stream, ln_small, n_launch)
        record("add_layernorm_f32_64x768", w.op, w.shape, w.dtype, True, ev, n_launch,
               {"note": "596 KB, cache resident and launch-latency bound; GB/s not an HBM figure"})

        # LayerNorm variants at the headline shape: ReLU, pre-norm sum and per-row statistics
        w = synth.WORKLOADS[HEADLINE]
        d = w.inputs()
        gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
        sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"], "s": d["x"]}, ROTATE_BYTES)
        stats = [(torch.empty(w.shape[0], device="cuda"), torch.empty(w.shape[0], device="cuda")) for _ in sets]

        def ln_ex(i):
            s, (m, v) = sets[i % len(sets)], stats[i % len(sets)]
            api.fuse_add_layernorm_ex(s["x"], s["r"], gamma, beta, d["eps"], relu=True, y=s["y"], sum_out=s["s"],
                                      mean_out=m, var_out=v)
        _, ev = time_launches(torch, stream, ln_ex, n_launch)
        record("add_layernorm_ex_relu_sum_stats_f16_2048x4096", "add_layernorm_ex", w.shape, w.dtype, True, ev,
               n_launch, {"note": "LayerNorm+ReLU with the pre-norm sum and fp32 mean/var also stored"})
        del sets, stats

        # bf16 I/O at the headline shape
        xb, rb = d["x"].bfloat16(), d["residual"].bfloat16()
        gb, bb = d["gamma"].bfloat16().cuda(), d["beta"].bfloat16().cuda()
        sets = rotation_sets(torch, {"x": xb, "r": rb}, {"y": xb}, ROTATE_BYTES)

        def ln_bf16(i):
            s = sets[i % len(sets)]
            api.fuse_add_layernorm(s["x"], s["r"], gb, bb, d["eps"], y=s["y"])
        _, ev = time_launches(torch, stream, ln_bf16, n_launch)
        record("add_layernorm_bf16_2048x4096", "add_layernorm", w.shape, "bf16", True, ev, n_launch)
        del sets

        w = synth.WORKLOADS["cumsum_f16_2048x4096"]
        d = w.inputs()
        sets = rotation_sets(torch, {"x": d["x"]}, {"y": d["x"]}, ROTATE_BYTES)
        ws = api._workspace(api.FUSE_OP_CUMSUM_SCALE, *w.shape, 0, api.FUSE_F16, "cuda")

        def cs(i):
            s = sets[i % len(sets)]
            api.fuse_cumsum_scale_rows(s["x"], d["scale"], y=s["y"])

        def cs_unf(i):
            s = sets[i % len(sets)]
            api.fuse_unfused_cumsum_scale_rows(s["x"], d["scale"], y=s["y"], workspace=ws)
        _, ev = time_launches(torch, stream, cs, n_launch)
        record("cumsum_scale_f16_2048x4096", w.op, w.shape, w.dtype, True, ev, n_launch)
        _, ev = time_launches(torch, stream, cs_unf, n_launch)
        record("cumsum_scale_unfused_f16_2048x4096", w.op, w.shape, w.dtype, False, ev, n_launch,
               {"note": "scan kernel storing the prefix sums + scale kernel"})
        del sets, ws

        w = synth.WORKLOADS["gelu_f16_2048x4096"]
        d = w.inputs()
        bias = d["bias"].cuda()
        sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"]}, ROTATE_BYTES)
        ws = api._workspace(api.FUSE_OP_BIAS_GELU_RESIDUAL, *w.shape, 0, api.FUSE_F16, "cuda")

        def gelu(i):
            s = sets[i % len(sets)]
            api.fuse_bias_gelu_residual(s["x"], bias, s["r"], y=s["y"])

        def gelu_unf(i):
            s = sets[i % len(sets)]
            api.fuse_unfused_bias_gelu_residual(s["x"], bias, s["r"], y=s["y"], workspace=ws)
        _, ev = time_launches(torch, stream, gelu, n_launch)
        record("bias_gelu_residual_f16_2048x4096", w.op, w.shape, w.dtype, True, ev, n_launch)
        _, ev = time_launches(torch, stream, gelu_unf, n_launch)
        record("bias_gelu_residual_unfused_f16_2048x4096", w.op, w.shape, w.dtype, False, ev, n_launch)
        del sets, ws

        w = synth.WORKLOADS["softmax_f16_65536x2048"]
        d = w.inputs()
        sets = rotation_sets(torch, {"x": d["x"]}, {"y": d["x"]}, ROTATE_BYTES)
        ws = api._workspace(api.FUSE_OP_SOFTMAX_ROWS, *w.shape, 0, api.FUSE_F16, "cuda")
        del d

        def sm(i):
            s = sets[i % len(sets)]
            api.fuse_softmax_rows(s["x"], 1 / math.sqrt(128), y=s["y"])

        def sm_unf(i):
            s = sets[i % len(sets)]
            api.fuse_unfused_softmax_rows(s["x"], 1 / math.sqrt(128), y=s["y"], workspace=ws)
        _, ev = time_launches(torch, stream, sm, n_launch // 2)
        record("softmax_f16_65536x2048", w.op, w.shape, w.dtype, True, ev, n_launch // 2)
        _, ev = time_launches(torch, stream, sm_unf, n_launch // 2)
        record("softmax_unfused_f16_65536x2048", w.op, w.shape, w.dtype, False, ev, n_launch // 2)
        del sets, ws

        ceiling = mfma_ceiling(torch, api, stream, roofline, MFMA_LAUNCHES)
        out["mfma_ceiling"] = ceiling

        w = synth.WORKLOADS["swiglu_bf16_2048x8960x1536"]
        d = w.inputs()
        a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
        o = torch.empty(w.shape[0], w.shape[1], dtype=torch.bfloat16, device="cuda")
        ws = api._workspace(api.FUSE_OP_SWIGLU, *w.shape, api.FUSE_BF16, "cuda")

        def sw(i):
            api.fuse_swiglu_dualgemm(a, b1, b2, out=o)

        def sw_unf(i):
            api.fuse_unfused_swiglu(a, b1, b2, out=o, workspace=ws)
        for i in range(3):
            sw(i)
        one = single_dispatch_us(torch, stream, sw)
        _, ev = time_launches(torch, stream, sw, MFMA_LAUNCHES)
        record("swiglu_bf16_2048x8960x1536", w.op, w.shape, w.dtype, True, ev, MFMA_LAUNCHES,
               single_dispatch(one, roofline.workload_work(w.op, w.shape, w.dtype, True)))
        of_ceiling("swiglu_bf16_2048x8960x1536", ceiling)
        _, ev = time_launches(torch, stream, sw_unf, MFMA_LAUNCHES)
        record("swiglu_unfused_bf16_2048x8960x1536", w.op, w.shape, w.dtype, False, ev, MFMA_LAUNCHES)
        del ws

        w = synth.WORKLOADS["gemm_relu_bf16_2048x8960x1536"]
        d = w.inputs()
        x, wt, bias = d["x"].cuda(), d["w"].cuda(), d["bias"].cuda()
        y = torch.empty(w.shape[0], w.shape[1], dtype=torch.bfloat16, device="cuda")
        ws = api._workspace(api.FUSE_OP_GEMM_BIAS_ACT, *w.shape, api.FUSE_BF16, "cuda")

        def gm(i):
            api.fuse_gemm_bias_act(x, wt, bias, "relu", y=y)

        def gm_unf(i):
            api.fuse_unfused_gemm_bias_act(x, wt, bias, "relu", y=y, workspace=ws)

        def gm_vendor(i):  # reference only: torch's library GEMM, not part of the path
            torch.matmul(x, wt, out=y)
        for i in range(3):
            gm(i)
        one = single_dispatch_us(torch, stream, gm)
        _, ev = time_launches(torch, stream, gm, MFMA_LAUNCHES)
        record("gemm_bias_relu_bf16_2048x8960x1536", w.op, w.shape, w.dtype, True, ev, MFMA_LAUNCHES,
               single_dispatch(one, roofline.workload_work(w.op, w.shape, w.dtype, True)))
        of_ceiling("gemm_bias_relu_bf16_2048x8960x1536", ceiling)
        _, ev = time_launches(torch, stream, gm_unf, MFMA_LAUNCHES)
        record("gemm_bias_relu_unfused_bf16_2048x8960x1536", w.op, w.shape, w.dtype, False, ev, MFMA_LAUNCHES,
               {"note": "GEMM kernel, bias kernel, ReLU kernel"})
        _, ev = time_launches(torch, stream, gm_vendor, MFMA_LAUNCHES)
        record("reference_vendor_gemm_bf16_2048x8960x1536", w.op, w.shape, w.dtype, True, ev, MFMA_LAUNCHES,
               {"note": "torch.matmul (hipBLASLt) without bias or activation: context for the MFMA ceiling, "
                        "not part of the path"})
        del ws

        # copy of the headline's byte count (read 32 MiB + write 16 MiB would not be a copy;
        # copy 24 MiB -> 24 MiB moves the same 48 MiB)
        nbytes = 24 << 20
        n = max(2, math.ceil(ROTATE_BYTES / (2 * nbytes)))
        bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
                 torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(n)]

        def cp(i):
            s, t = bufs[i % len(bufs)]
            api.fuse_copy(s, t)
        _, ev = time_launches(torch, stream, cp, n_launch)
        us = ev * 1e3 / n_launch
        gb = 2 * nbytes / (us * 1e-6) / 1e9
        out["copy_48MiB"] = {"avg_launch_us": round(us, 3), "achieved_gbps": round(gb, 1),
                             "frac": round(gb / peak_bw, 4), "bound": "hbm",
                             "note": "plain copy of 24 MiB (48 MiB moved): the achievable streaming ceiling"}
        log(f"copy: {us:.2f} us {gb:.0f} GB/s")
        del bufs

        # the same ceiling at the softmax's size (256 MiB read, 256 MiB written)
        nbytes = 256 << 20
        bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
                 torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(3)]

        def cp_big(i):
            s, t = bufs[i % len(bufs)]
            api.fuse_copy(s, t)
        _, ev = time_launches(torch, stream, cp_big, n_launch // 2)
        us = ev * 1e3 / (n_launch // 2)
        gb = 2 * nbytes / (us * 1e-6) / 1e9
        out["copy_512MiB"] = {"avg_launch_us": round(us, 3), "achieved_gbps": round(gb, 1),
                              "frac": round(gb / peak_bw, 4), "bound": "hbm",
                              "note": "plain copy of 256 MiB (512 MiB moved): the ceiling at the softmax's size"}
        log(f"copy 512 MiB: {us:.2f} us {gb:.0f} GB/s")
        del bufs
    return out


CEILING_ITERS = 448  # rounds of the matrix-core calibration kernel: about the SwiGLU workload's length
# Launches per back-to-back replay of the matrix-core rows and their ceiling.  Under the board's
# power limit the clock oscillates over a few milliseconds: consecutive replays of 20 SwiGLU
# launches measured 110-142 us per launch on one box, one of 200 launches 118.8 us each time.
MFMA_LAUNCHES = 200


def mfma_ceiling(torch, api, stream, roofline, n_launch, iters=CEILING_ITERS):
    """The matrix-core calibration kernel (bf16 32x32x16 MFMAs from registers, two workgroups of
    four waves per CU) sized to run about as long as the SwiGLU workload, timed the two ways the
    matrix-core rows are: one synchronised dispatch at a time, and back to back."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    flops = wgs * 4 * iters * 8 * 32768
    res = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")

    def run(i):
        api.fuse_mfma_ceiling(wgs, iters, res)
    for i in range(3):
        run(i)
    one = single_dispatch_us(torch, stream, run)
    _, ev = time_launches(torch, stream, run, n_launch)
    us = ev * 1e3 / n_launch
    peak = roofline.MFMA_PEAK_TFLOPS["bf16"]
    tf1, tf = flops / (one * 1e-6) / 1e12, flops / (us * 1e-6) / 1e12
    log(f"mfma ceiling: {one:.2f} us single ({tf1:.0f} TFLOP/s), {us:.2f} us back to back ({tf:.0f} TFLOP/s)")
    return {"workgroups": wgs, "iters": iters, "flops": flops,
            "single_dispatch_us": round(one, 3), "single_dispatch_tflops": round(tf1, 1),
            "avg_launch_us": round(us, 3), "achieved_tflops": round(tf, 1),
            "frac_of_peak": {"single_dispatch": round(tf1 / peak, 4), "back_to_back": round(tf / peak, 4)},
            "note": "fuse_mfma_ceiling: only bf16 matrix-core instructions, operands in registers, no memory "
                    "traffic; the rate the matrix cores sustain on this part, against which the matrix-core "
                    "rows' frac_of_mfma_ceiling is taken (their roofline frac stays against the spec peak)"}


SWEEP_ROWS = (512, 1024, 2048, 4096, 8192, 16384, 32768)


def linear_fit(xs, ys):
    """Least-squares line y = a + b x; returns (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    return my - b * mx, b


def size_sweep(torch, api, synth, roofline, n=40):
    """Fused Add+LayerNorm fp16 at H = 4096 and a plain copy of the same byte count, over rows
    512 ... 32768, cold (each launch on a buffer set not touched for 1 GiB of traffic), each size
    replayed n times from a HIP graph.  A line t = t0 + bytes / bw fitted to each kernel's times
    separates the fixed cost per launch (t0) from the streaming rate it approaches (bw).  Under
    rocprofv3 --kernel-trace every size is a grid of its own, so the trace gives the same sweep in
    kernel durations."""
    w = synth.WORKLOADS[HEADLINE]
    base = w.inputs()
    hidden = w.shape[1]
    bx, br = base["x"].cuda(), base["residual"].cuda()
    gamma, beta = base["gamma"].cuda(), base["beta"].cuda()
    stream = torch.cuda.Stream()
    sizes = []

    def rows_of(t, rows):
        return t[:rows].clone() if rows <= t.shape[0] else t.repeat(rows // t.shape[0], 1)

    with torch.cuda.stream(stream):
        for rows in SWEEP_ROWS:
            work = roofline.workload_work("add_layernorm", (rows, hidden), "f16")
            per_set = 3 * rows * hidden * 2
            nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
            sets = [(rows_of(bx, rows), rows_of(br, rows), torch.empty(rows, hidden, dtype=torch.float16, device="cuda"))
                    for _ in range(nsets)]

            def ln(i):
                x, r, y = sets[i % nsets]
                api.fuse_add_layernorm(x, r, gamma, beta, 1e-5, y=y)
            _, ev = time_launches(torch, stream, ln, n)
            ln_us = ev * 1e3 / n
            del sets
            nbytes = 3 * rows * hidden  # a copy of this many bytes moves the three tensors' bytes
            nb = max(2, math.ceil(ROTATE_BYTES / (2 * nbytes)))
            bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
                     torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(nb)]

            def cp(i):
                s, t = bufs[i % nb]
                api.fuse_copy(s, t)
            _, ev = time_launches(torch, stream, cp, n)
            cp_us = ev * 1e3 / n
            del bufs
            sizes.append({"rows": rows, "bytes": work["bytes"], "add_layernorm_us": round(ln_us, 3),
                          "copy_us": round(cp_us, 3), "copy_bytes": 2 * nbytes,
                          "add_layernorm_frac": round(work["bytes"] / (ln_us * 1e-6) / 1e9 / roofline.HBM_PEAK_GBPS, 4),
                          "copy_frac": round(2 * nbytes / (cp_us * 1e-6) / 1e9 / roofline.HBM_PEAK_GBPS, 4)})
            log(f"sweep rows={rows}: add_layernorm {ln_us:.2f} us, copy {cp_us:.2f} us")
    out = {"hidden": hidden, "dtype": "f16", "launches_per_size": n, "timing": "HIP events around a graph replay",
           "sizes": sizes}
    for key, bkey in (("add_layernorm", "bytes"), ("copy", "copy_bytes")):
        t0, inv_bw = linear_fit([s[bkey] for s in sizes], [s[f"{key}_us"] for s in sizes])
        out[f"{key}_fit"] = {"t0_us": round(t0, 3), "bw_gbps": round(1e-3 / inv_bw, 1),
                             "bw_frac": round(1e-3 / inv_bw / roofline.HBM_PEAK_GBPS, 4)}
    return out


def counters_pass(torch, api, synth, n=8):
    """A few eager dispatches of each kernel whose HBM bytes the hardware counters are read for
    (run under rocprofv3 --pmc): fused Add+LayerNorm, its unfused chain, the fused and unfused
    GELU chain, and a copy of exactly 24 MiB (48 MiB moved) as the calibration of the counters.
    Every dispatch uses a buffer set not touched for more than 1 GiB of traffic."""
    w = synth.WORKLOADS[HEADLINE]
    d = w.inputs()
    gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
    sets = rotation_sets(torch, {"x": d["x"], "r": d["residual"]}, {"y": d["x"]}, ROTATE_BYTES)
    ws = api._workspace(api.FUSE_OP_ADD_LAYERNORM, *w.shape, 0, api.FUSE_F16, "cuda")
    bias = d["beta"].cuda()
    wsg = api._workspace(api.FUSE_OP_BIAS_GELU_RESIDUAL, *w.shape, 0, api.FUSE_F16, "cuda")
    nbytes = 24 << 20
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(len(sets))]
    k = 0
    for name, fn in (
        ("add_layernorm", lambda s: api.fuse_add_layernorm(s["x"], s["r"], gamma, beta, 1e-5, y=s["y"])),
        ("add_layernorm_unfused", lambda s: api.fuse_unfused_add_layernorm(s["x"], s["r"], gamma, beta, 1e-5,
                                                                           y=s["y"], workspace=ws)),
        ("bias_gelu_residual", lambda s: api.fuse_bias_gelu_residual(s["x"], bias, s["r"], y=s["y"])),
        ("bias_gelu_residual_unfused", lambda s: api.fuse_unfused_bias_gelu_residual(s["x"], bias, s["r"],
                                                                                     y=s["y"], workspace=wsg)),
    ):
        for _ in range(n):
            fn(sets[k % len(sets)])
            k += 1
            torch.cuda.synchronize()
        log(f"counters: {n} x {name}")
    for i in range(n):
        s, t = bufs[(i + 7) % len(bufs)]
        api.fuse_copy(s, t)
        torch.cuda.synchronize()
    log(f"counters: {n} x copy of {nbytes} bytes")


def counters_rows(torch, api, synth, n=4):
    """Like counters_pass for the other rows of the path: a few cold dispatches (1 GiB rotation)
    of each fused kernel and its unfused chain, then the 24 MiB copy calibration."""
    def run(name, inputs, outputs, fn):
        sets = rotation_sets(torch, inputs, outputs, ROTATE_BYTES)
        for i in range(n):
            fn(sets[i % len(sets)])
            torch.cuda.synchronize()
        log(f"counters: {n} x {name}")
        del sets

    w = synth.WORKLOADS[HEADLINE]
    d = w.inputs()
    gamma, beta = d["gamma"].cuda(), d["beta"].cuda()
    stats = (torch.empty(w.shape[0], device="cuda"), torch.empty(w.shape[0], device="cuda"))
    run("add_layernorm_ex", {"x": d["x"], "r": d["residual"]}, {"y": d["x"], "s": d["x"]},
        lambda s: api.fuse_add_layernorm_ex(s["x"], s["r"], gamma, beta, 1e-5, relu=True, y=s["y"], sum_out=s["s"],
                                            mean_out=stats[0], var_out=stats[1]))
    w = synth.WORKLOADS["cumsum_f16_2048x4096"]
    d = w.inputs()
    ws = api._workspace(api.FUSE_OP_CUMSUM_SCALE, *w.shape, 0, api.FUSE_F16, "cuda")
    run("cumsum_scale", {"x": d["x"]}, {"y": d["x"]}, lambda s: api.fuse_cumsum_scale_rows(s["x"], d["scale"], y=s["y"]))
    run("cumsum_scale_unfused", {"x": d["x"]}, {"y": d["x"]},
        lambda s: api.fuse_unfused_cumsum_scale_rows(s["x"], d["scale"], y=s["y"], workspace=ws))
    del ws
    w = synth.WORKLOADS["softmax_f16_65536x2048"]
    d = w.inputs()
    ws = api._workspace(api.FUSE_OP_SOFTMAX_ROWS, *w.shape, 0, api.FUSE_F16, "cuda")
    run("softmax", {"x": d["x"]}, {"y": d["x"]}, lambda s: api.fuse_softmax_rows(s["x"], d["scale"], y=s["y"]))
    run("softmax_unfused", {"x": d["x"]}, {"y": d["x"]},
        lambda s: api.fuse_unfused_softmax_rows(s["x"], d["scale"], y=s["y"], workspace=ws))
    del ws, d
    w = synth.WORKLOADS["swiglu_bf16_2048x8960x1536"]
    d = w.inputs()
    M, N, K = w.shape
    o = torch.empty(M, N, dtype=torch.bfloat16)
    ws = api._workspace(api.FUSE_OP_SWIGLU, M, N, K, api.FUSE_BF16, "cuda")
    io = {"a": d["a"], "b1": d["b1"], "b2": d["b2"]}
    run("swiglu", io, {"o": o}, lambda s: api.fuse_swiglu_dualgemm(s["a"], s["b1"], s["b2"], out=s["o"]))
    run("swiglu_unfused", io, {"o": o},
        lambda s: api.fuse_unfused_swiglu(s["a"], s["b1"], s["b2"], out=s["o"], workspace=ws))
    del ws, d
    w = synth.WORKLOADS["gemm_relu_bf16_2048x8960x1536"]
    d = w.inputs()
    ws = api._workspace(api.FUSE_OP_GEMM_BIAS_ACT, M, N, K, api.FUSE_BF16, "cuda")
    io = {"x": d["x"], "w": d["w"], "b": d["bias"]}
    run("gemm_bias_relu", io, {"y": o}, lambda s: api.fuse_gemm_bias_act(s["x"], s["w"], s["b"], "relu", y=s["y"]))
    run("gemm_bias_relu_unfused", io, {"y": o},
        lambda s: api.fuse_unfused_gemm_bias_act(s["x"], s["w"], s["b"], "relu", y=s["y"], workspace=ws))
    del ws, d
    nbytes = 24 << 20
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(22)]
    for i in range(8):
        s, t = bufs[(i + 7) % len(bufs)]
        api.fuse_copy(s, t)
        torch.cuda.synchronize()
    log(f"counters: 8 x copy of {nbytes} bytes")


def dispatch_only(torch, api, synth, name, count):
    """`count` eager dispatches of one fused row at its workload (for a profiler run), no timing.
    `mfma_ceiling` dispatches the matrix-core calibration kernel as the benchmark sizes it."""
    if name == "mfma_ceiling":
        wgs = 2 * torch.cuda.get_device_properties(0).multi_processor_count
        res = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        for _ in range(count):
            api.fuse_mfma_ceiling(wgs, CEILING_ITERS, res)
            torch.cuda.synchronize()
        log(f"dispatched {count} x mfma_ceiling ({wgs} workgroups, {CEILING_ITERS} rounds)")
        return
    w = synth.WORKLOADS[name]
    d = {k: (v.cuda() if hasattr(v, "cuda") else v) for k, v in w.inputs().items()}
    if w.op == "swiglu":
        call = lambda: api.fuse_swiglu_dualgemm(d["a"], d["b1"], d["b2"])
    elif w.op == "gemm_bias_act":
        call = lambda: api.fuse_gemm_bias_act(d["x"], d["w"], d["bias"], "relu")
    elif w.op == "softmax_rows":
        call = lambda: api.fuse_softmax_rows(d["x"], d["scale"])
    elif w.op == "cumsum_scale_rows":
        call = lambda: api.fuse_cumsum_scale_rows(d["x"], d["scale"])
    elif w.op == "bias_gelu_residual":
        call = lambda: api.fuse_bias_gelu_residual(d["x"], d["bias"], d["residual"])
    else:
        call = lambda: api.fuse_add_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], d["eps"])
    for _ in range(count):
        call()
        torch.cuda.synchronize()
    log(f"dispatched {count} x {name}")


def launch_study(torch, api, synth, n_empty=4000, n_graph=1000, n_steps=200):
    """Launch cost on this GPU ([P2] §4.5, [P3] §2): an empty kernel enqueued from a loop inside
    the library (host cost per call, back-to-back interval on the GPU, cost per kernel inside a
    replayed graph), and small latency-bound rows fused vs unfused, host-launched from Python vs
    replayed from a graph."""
    stream = torch.cuda.Stream()
    out = {}
    with torch.cuda.stream(stream):
        api.fuse_empty_kernels(200)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        api.fuse_empty_kernels(n_empty)
        t1 = time.perf_counter()
        e1.record(stream)
        torch.cuda.synchronize()
        out["empty_kernel_host_enqueue_us"] = round((t1 - t0) * 1e6 / n_empty, 3)
        out["empty_kernel_back_to_back_us"] = round(e0.elapsed_time(e1) * 1e3 / n_empty, 3)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            api.fuse_empty_kernels(n_graph)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out["empty_kernel_in_graph_us"] = round(e0.elapsed_time(e1) * 1e3 / n_graph, 3)
        del g

        def steps(name, launch, kernels):
            for i in range(3):
                launch(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n_steps):
                launch(i)
            torch.cuda.synchronize()
            eager = (time.perf_counter() - t0) * 1e6 / n_steps
            _, ev = time_launches(torch, stream, launch, n_steps)
            out[name] = {"kernels_per_step": kernels, "eager_python_us_per_step": round(eager, 2),
                         "graph_us_per_step": round(ev * 1e3 / n_steps, 3)}
            log(f"{name}: eager {eager:.1f} us, graph {ev * 1e3 / n_steps:.2f} us per step")

        d = synth.WORKLOADS["addln_f32_64x768"].inputs()
        g_ = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
        y = torch.empty_like(g_["x"])
        ws = api._workspace(api.FUSE_OP_ADD_LAYERNORM, 64, 768, 0, api.FUSE_F32, "cuda")
        steps("add_layernorm_f32_64x768_fused",
              lambda i: api.fuse_add_layernorm(g_["x"], g_["residual"], g_["gamma"], g_["beta"], d["eps"], y=y), 1)
        steps("add_layernorm_f32_64x768_unfused",
              lambda i: api.fuse_unfused_add_layernorm(g_["x"], g_["residual"], g_["gamma"], g_["beta"], d["eps"],
                                                       y=y, workspace=ws), 2)
        d = synth.bias_gelu_residual_inputs(64, 4096, "f16", 1002)
        g_ = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
        y = torch.empty_like(g_["x"])
        ws = api._workspace(api.FUSE_OP_BIAS_GELU_RESIDUAL, 64, 4096, 0, api.FUSE_F16, "cuda")
        steps("bias_gelu_residual_f16_64x4096_fused",
              lambda i: api.fuse_bias_gelu_residual(g_["x"], g_["bias"], g_["residual"], y=y), 1)
        steps("bias_gelu_residual_f16_64x4096_unfused",
              lambda i: api.fuse_unfused_bias_gelu_residual(g_["x"], g_["bias"], g_["residual"], y=y, workspace=ws), 3)
    log(f"empty kernel: host {out['empty_kernel_host_enqueue_us']} us, back-to-back "
        f"{out['empty_kernel_back_to_back_us']} us, in graph {out['empty_kernel_in_graph_us']} us")
    return out


def interleaved(torch, stream, variants, n, rounds):
    """Times several variants against each other without an order bias: each variant is captured
    as a graph of n launches, then `rounds` rounds replay every graph once, the starting variant
    rotating from round to round (ABCD, BCDA, ...), so the clock's drift under the power limit
    and the caches left by the previous variant fall on every variant alike.  Returns, per
    variant, the median, minimum and maximum over the rounds of the time per launch (us)."""
    graphs = {}
    for name, f in variants.items():
        for i in range(3):
            f(i)
        torch.cuda.synchronize()
        graphs[name] = Timed(torch, stream, f, n)
        graphs[name].run()
    names = list(graphs)
    times = {k: [] for k in names}
    for r in range(rounds):
        for j in range(len(names)):
            k = names[(r + j) % len(names)]
            _, ev = graphs[k].run()
            times[k].append(ev * 1e3 / n)
    return {k: {"median_us": round(statistics.median(v), 2), "min_us": round(min(v), 2), "max_us": round(max(v), 2)}
            for k, v in times.items()}


def selection_study(torch, api, synth, K=1536, n=20, rounds=5):
    """Fused (scheme B) against unfused (scheme A) SwiGLU over shapes ([P4] 不同场景下的选型建议
    derives its thresholds from block counts against SM counts): this library's own scheme A
    (the product kernel storing c1 and c2, then SiLU * product), its per-shape plan (the fused
    kernel or its split-K form) and, for context, the library-GEMM form of scheme A (two torch
    matmuls, then SiLU and product as torch kernels).  Same buffers every launch (the weights stay
    cache-resident, as they would across a model's layers).  The four are timed interleaved (see
    `interleaved`); a ratio between two of them is marked significant only when their ranges over
    the rounds do not overlap."""
    import torch.nn.functional as F
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.Stream()
    out = {"cus": cus, "K": K, "launches_per_replay": n, "rounds": rounds,
           "timing": "median (min..max) over interleaved rounds of a graph replay", "shapes": []}
    with torch.cuda.stream(stream):
        for M in (256, 1024, 2048):
            for N in (256, 512, 1024, 2048, 4096, 8960):
                d = synth.swiglu_inputs(M, N, K, "bf16", seed=M + N)
                a, b1, b2 = d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()
                o = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
                c1, c2 = torch.empty_like(o), torch.empty_like(o)
                ws = api._workspace(api.FUSE_OP_SWIGLU, M, N, K, api.FUSE_BF16, "cuda")
                wsa = api._auto_workspace(api.FUSE_OP_SWIGLU, M, N, K, "cuda")

                def lib_a(i):
                    torch.matmul(a, b1, out=c1)
                    torch.matmul(a, b2, out=c2)
                    torch.mul(F.silu(c1), c2, out=o)
                variants = {
                    "fused": lambda i: api.fuse_swiglu_dualgemm(a, b1, b2, out=o),
                    "unfused": lambda i: api.fuse_unfused_swiglu(a, b1, b2, out=o, workspace=ws),
                    "auto": lambda i: api.fuse_swiglu_auto(a, b1, b2, out=o, workspace=wsa),
                    "library_gemm_scheme_a": lib_a,
                }
                t = interleaved(torch, stream, variants, n, rounds)
                r = {"M": M, "N": N, "tiles_fused": -(-M // 256) * -(-N // 128),
                     "auto_splits": api.fuse_auto_splits(api.FUSE_OP_SWIGLU, M, N, K), "times": t}
                for a_, b_ in (("unfused", "fused"), ("fused", "auto"), ("library_gemm_scheme_a", "auto")):
                    ratio = t[a_]["median_us"] / t[b_]["median_us"]
                    apart = t[a_]["min_us"] > t[b_]["max_us"] or t[b_]["min_us"] > t[a_]["max_us"]
                    r[f"{a_}_over_{b_}"] = {"ratio": round(ratio, 3), "significant": apart}
                out["shapes"].append(r)
                log(f"selection M={M} N={N}: " + ", ".join(f"{k} {v['median_us']} ({v['min_us']}..{v['max_us']})"
                                                          for k, v in t.items()) + f" us; {r['auto_splits']} splits")
                del ws, wsa
    return out


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, roofline, budget_s=8.0, single_budget_s=4.0):
    """The oracle timed on the host: all OpenMP threads for about budget_s, then one thread for
    about single_budget_s, on the full headline workload."""
    import numpy as np

    import oracle

    w = synth.WORKLOADS[HEADLINE]
    d = w.inputs()
    x, r, g, b = (oracle.f64(d[k]) for k in ("x", "residual", "gamma", "beta"))
    eps = float(np.float32(d["eps"]))
    work = roofline.workload_work(w.op, w.shape, w.dtype)

    def run(budget):
        oracle.add_layernorm(x, r, g, b, eps)  # warm (page faults, library load, thread pool)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.add_layernorm(x, r, g, b, eps)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 100000:
                return reps, el

    threads = oracle.threads()
    reps, el = run(budget_s)
    per = el / reps
    oracle.set_threads(1)
    try:
        reps1, el1 = run(single_budget_s)
    finally:
        oracle.set_threads(threads)
    per1 = el1 / reps1
    # the product path's result on the same inputs against the oracle's
    import torch
    from oracle.tolerance import RULE_TEXT, compare

    from memory_bound_amd import api
    y = api.fuse_add_layernorm(d["x"].cuda(), d["residual"].cuda(), d["gamma"].cuda(), d["beta"].cuda(), d["eps"])
    c = compare(y, oracle.add_layernorm(x, r, g, b, eps), w.dtype)
    par = {"rule": RULE_TEXT[w.dtype], "n": c["n"], "max_abs_err": c["max_abs"],
           "max_err_over_allowed": round(c["max_excess"], 4), "n_bad": c["n_bad"], "ok": c["ok"]}
    torch.cuda.synchronize()
    return {"value": round(work["bytes"] / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"full {w.shape[0]}x{w.shape[1]} workload, {reps} oracle calls in {el:.1f} s "
                      f"({per * 1e3:.2f} ms per call, fp64, inputs pre-widened)",
            "single_thread": {"value": round(work["bytes"] / per1 / 1e9, 3), "unit": "GB/s",
                              "sample": f"{reps1} calls in {el1:.1f} s ({per1 * 1e3:.2f} ms per call)"},
            "host_cpu": host_cpu_model(), "host_cpus": os.cpu_count(), "parity": par}


# (workload, rows of it in the timed sample) for the oracle timings of the other rows: whole
# workloads where one oracle call takes well under the budget, leading rows otherwise
CPU_ROWS = (("addln_f32_64x768", None), ("gelu_f16_2048x4096", None), ("addln_f16_16384x4096", 2048),
            ("softmax_f16_65536x2048", 4096), ("cumsum_f16_2048x4096", None),
            ("swiglu_bf16_2048x8960x1536", 8), ("gemm_relu_bf16_2048x8960x1536", 8))


def cpu_rows(synth, roofline, budget_s=1.0):
    """The oracle timed on the host for every other workload, all OpenMP threads and then one
    thread, about budget_s each, on the whole workload or its leading rows (the row work of these
    operations is independent, so a row sample scales)."""
    import numpy as np

    import oracle

    def timed(fn, budget):
        fn()  # warm
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return el / reps

    import torch
    from oracle.tolerance import RULE_TEXT, compare

    from memory_bound_amd import api

    def parity(y_gpu, ref, kind, rows):
        # the product path's result on the same inputs, its leading rows against the oracle's
        y = y_gpu if rows is None else y_gpu[:rows]
        r = compare(y, ref, kind)
        return {"rule": RULE_TEXT[kind], "n": r["n"], "max_abs_err": r["max_abs"],
                "max_err_over_allowed": round(r["max_excess"], 4), "n_bad": r["n_bad"], "ok": r["ok"]}

    out = {}
    threads = oracle.threads()
    for name, rows in CPU_ROWS:
        w = synth.WORKLOADS[name]
        d = w.inputs()
        shape = w.shape if rows is None else (rows,) + tuple(w.shape[1:])
        cut = (lambda t: t) if rows is None else (lambda t: t[:rows])
        g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
        if w.op == "add_layernorm":
            x, r, gm, b = oracle.f64(cut(d["x"])), oracle.f64(cut(d["residual"])), oracle.f64(d["gamma"]), \
                oracle.f64(d["beta"])
            eps = float(np.float32(d["eps"]))
            fn = lambda: oracle.add_layernorm(x, r, gm, b, eps)
            gpu = lambda: api.fuse_add_layernorm(g["x"], g["residual"], g["gamma"], g["beta"], d["eps"])
        elif w.op == "bias_gelu_residual":
            x, bias, r = oracle.f64(cut(d["x"])), oracle.f64(d["bias"]), oracle.f64(cut(d["residual"]))
            fn = lambda: oracle.bias_gelu_residual(x, bias, r)
            gpu = lambda: api.fuse_bias_gelu_residual(g["x"], g["bias"], g["residual"])
        elif w.op == "softmax_rows":
            x, sc = oracle.f64(cut(d["x"])), float(np.float32(d["scale"]))
            fn = lambda: oracle.softmax_rows(x, sc)
            gpu = lambda: api.fuse_softmax_rows(g["x"], d["scale"])
        elif w.op == "cumsum_scale_rows":
            x, sc = oracle.f64(cut(d["x"])), float(np.float32(d["scale"]))
            fn = lambda: oracle.cumsum_scale_rows(x, sc)
            gpu = lambda: api.fuse_cumsum_scale_rows(g["x"], d["scale"])
        elif w.op == "swiglu":
            a, b1, b2 = oracle.f64(cut(d["a"])), oracle.f64(d["b1"]), oracle.f64(d["b2"])
            fn = lambda: oracle.swiglu(a, b1, b2)
            gpu = lambda: api.fuse_swiglu_dualgemm(g["a"], g["b1"], g["b2"])
        else:
            x, wt, bias = oracle.f64(cut(d["x"])), oracle.f64(d["w"]), oracle.f64(d["bias"])
            fn = lambda: oracle.gemm_bias_act(x, wt, bias, "relu")
            gpu = lambda: api.fuse_gemm_bias_act(g["x"], g["w"], g["bias"], "relu")
        work = roofline.workload_work(w.op, shape, w.dtype)
        per = timed(fn, budget_s)
        oracle.set_threads(1)
        try:
            per1 = timed(fn, budget_s)
        finally:
            oracle.set_threads(threads)
        if "flops" in work:
            val, val1, unit = work["flops"] / per / 1e12, work["flops"] / per1 / 1e12, "TFLOP/s"
        else:
            val, val1, unit = work["bytes"] / per / 1e9, work["bytes"] / per1 / 1e9, "GB/s"
        out[name] = {"value": round(val, 4), "single_thread": round(val1, 4), "unit": unit, "cores": threads,
                     "ms_per_call": round(per * 1e3, 3), "single_thread_ms_per_call": round(per1 * 1e3, 3),
                     "sample": "whole workload" if rows is None else f"leading {rows} of {w.shape[0]} rows",
                     "parity": parity(gpu(), fn(), w.dtype, rows)}
        log(f"oracle {name}: {val:.4g} {unit} on {threads} threads, {val1:.4g} on one")
    return out


SPLIT_SWEEP_SHAPES = (
    ("swiglu", 256, 512, 1536), ("swiglu", 256, 2048, 1536), ("swiglu", 512, 2048, 1536),
    ("swiglu", 1024, 1024, 1024), ("swiglu", 256, 4096, 4096), ("swiglu", 1024, 2048, 2048),
    ("swiglu", 2048, 1024, 4096), ("gemm", 1024, 1024, 1024), ("gemm", 256, 8960, 1536),
    ("gemm", 512, 4096, 4096), ("gemm", 2048, 2048, 2048), ("gemm", 2048, 2560, 2048),
    ("gemm", 2048, 2048, 512),
)
SPLIT_SWEEP_COUNTS = (1, 2, 3, 4, 5, 6, 8, 12)


def split_sweep(torch, api):
    """The split-K plan against every forced split count (FUSE_SPLITK) at the shapes its cost model
    was fitted to: per synchronised single dispatch of the auto entry points (median of 10), the
    time of each split count and of the plan's own choice."""
    stream = torch.cuda.Stream()
    out = []
    with torch.cuda.stream(stream):
        for op, M, N, K in SPLIT_SWEEP_SHAPES:
            g = torch.Generator().manual_seed(M + N + K)
            a = torch.randn(M, K, generator=g).to(torch.bfloat16).cuda()
            b1 = (torch.randn(K, N, generator=g) / math.sqrt(K)).to(torch.bfloat16).cuda()
            b2 = (torch.randn(K, N, generator=g) / math.sqrt(K)).to(torch.bfloat16).cuda()
            bias = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16).cuda()
            o = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            code = api.FUSE_OP_SWIGLU if op == "swiglu" else api.FUSE_OP_GEMM_BIAS_ACT
            kt = K // 32

            def timed():
                need = api.load().fuse_auto_workspace_bytes(code, M, N, K, api.FUSE_BF16)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
                if op == "swiglu":
                    f = lambda i: api.fuse_swiglu_auto(a, b1, b2, out=o, workspace=ws)
                else:
                    f = lambda i: api.fuse_gemm_bias_act_auto(a, b1, bias, "relu", y=o, workspace=ws)
                for i in range(3):
                    f(i)
                return round(single_dispatch_us(torch, stream, f), 2)
            r = {"op": op, "shape": [M, N, K], "forced": {}}
            for sp in SPLIT_SWEEP_COUNTS:
                if sp > kt:
                    continue
                os.environ["FUSE_SPLITK"] = str(sp)
                try:
                    r["forced"][str(api.fuse_auto_splits(code, M, N, K))] = timed()
                finally:
                    del os.environ["FUSE_SPLITK"]
            r["plan_splits"] = api.fuse_auto_splits(code, M, N, K)
            r["plan_us"] = timed()
            best = min(r["forced"], key=r["forced"].get)
            r["best_forced"] = [int(best), r["forced"][best]]
            log(f"split sweep {op} {M}x{N}x{K}: plan {r['plan_splits']} splits {r['plan_us']} us; "
                f"best forced {best} splits {r['forced'][best]} us; all {r['forced']}")
            out.append(r)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-rows", action="store_true", help="skip the other rows of the hot path")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--counters", action="store_true",
                    help="only run the short dispatch sequence read by rocprofv3 --pmc, no timing")
    ap.add_argument("--dispatch", metavar="WORKLOAD",
                    help="only dispatch the fused kernel of one workload (or mfma_ceiling, the matrix-core "
                         "calibration kernel) --dispatch-count times (profiling)")
    ap.add_argument("--dispatch-count", type=int, default=3)
    ap.add_argument("--counters-rows", action="store_true",
                    help="the same for the other rows of the path (their fused and unfused kernels)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the size sweep of fused Add+LayerNorm and the copy (fixed cost and streaming rate)")
    ap.add_argument("--split-sweep", action="store_true",
                    help="only the split-K plan against every forced split count (its fitted shapes)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the fused row kernels are "
              "single-GPU; rows shard across GPUs with no exchange, so N GPUs would run the same "
              "kernel on rows/N each.", file=sys.stderr)
        sys.exit(2)

    import torch

    from memory_bound_amd import api, roofline, synth

    api.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.counters:
        counters_pass(torch, api, synth)
        return
    if a.counters_rows:
        counters_rows(torch, api, synth)
        return
    if a.dispatch:
        dispatch_only(torch, api, synth, a.dispatch, a.dispatch_count)
        return
    if a.sweep:
        print(json.dumps({"size_sweep": size_sweep(torch, api, synth, roofline)}), flush=True)
        return
    if a.split_sweep:
        print(json.dumps({"split_sweep": split_sweep(torch, api)}), flush=True)
        return
    h = headline(torch, api, synth, roofline, a.steps, a.warmup)
    log(f"headline: {h['avg_launch_us']:.2f} us/launch, value {h['value_gbps']:.0f} GB/s")
    rows = {} if a.no_rows else other_rows(torch, api, synth, roofline)
    study = None if a.no_rows else launch_study(torch, api, synth)
    selection = None if a.no_rows else selection_study(torch, api, synth)
    cpu = None if a.no_cpu else cpu_baseline(synth, roofline)
    oracle_rows = None if (a.no_cpu or a.no_rows) else cpu_rows(synth, roofline)

    traffic, unfused_ratio = read_counters()
    trace = read_trace(h["bytes"])
    w = h["workload"]
    host_us, ev_us = h["host_s"] * 1e6, h["avg_launch_us"] * a.steps
    line = {
        "metric": "achieved HBM GB/s (% of peak) fused Add+LayerNorm [2048,4096] fp16",
        "value": round(h["value_gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(h["host_s"] * 1e3 / a.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # the arithmetic of the path; the tensors are stored as fp16 (config.storage)
        "data": "synthetic",
        "config": {"workload": "fused ResidualAdd+LayerNorm, [B,S,H]=[1,2048,4096] fp16, eps=1e-5",
                   "rows": w.shape[0], "hidden": w.shape[1], "storage": "f16", "seed": w.seed,
                   "buffer_sets": h["sets"], "launch": "HIP graph of the timed steps"},
        "pct_of_peak": round(100 * h["value_gbps"] / roofline.HBM_PEAK_GBPS, 2),
        "timing": {"host_wall_us": round(host_us, 2), "event_us": round(ev_us, 2),
                   "host_overhead_us": round(host_us - ev_us, 2),
                   "note": "value = algorithmic bytes x steps / host_wall_us (synchronised on both sides); "
                           "host_overhead_us is what the host adds once per timed region (graph launch and "
                           "synchronisation) over the HIP-event time of the same replay"},
        "roofline": {"bound": "hbm", "achieved": round(h["achieved_gbps"], 1),
                     "peak": roofline.HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(h["achieved_gbps"] / roofline.HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": h["bytes"],
                     "unfused_over_fused_traffic": unfused_ratio,
                     "avg_launch_us": round(h["avg_launch_us"], 3),
                     "definition": "achieved = algorithmic bytes / avg_launch_us, the HIP-event time of the "
                                   "timed graph replay on the launch stream over the steps: the kernel plus the "
                                   "dispatch gap to the next one.  kernel_trace: the same kernel's durations "
                                   "alone, from the committed rocprofv3 trace of this command",
                     "kernel_trace": trace},
        "cpu_baseline": cpu,
        "cpu_rows": oracle_rows,
        "headline_hot_cache": h["hot"],
        "rows": rows,
        "launch_study": study,
        "selection_study": selection,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
