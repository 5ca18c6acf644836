"""Benchmark: GEMM TFLOP/s of the pipelined MFMA kernel at 8192^3 on one MI355X, and the
fraction of the dense fp16/bf16 MFMA peak.

Headline workload (one "step" = one GEMM over inputs already resident in HBM): fp16
M = N = K = 8192, A [M,K] and B [K,N] row-major (NN), entries uniform [-1, 1] from seeds
42/43, fp32 accumulation, fp16 output -- the metric names fp16 8192^3; layout and inputs
are those of the 8192^3 configuration, which is bf16 and is reported under "extra"
beside every other configuration (256^3, 4096^3, 3000x5000x1000 with masked tails,
3072x4096x4096 with the fused GELU), each with its roofline and its oracle on the host.
Prints one JSON line.

  python bench.py [--gpus 1] [--steps 200] [--warmup 500] [--min-warmup-s 1.0]
                  [--no-cpu-baseline] [--no-extra]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense MFMA, published
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20                            # MI355X Infinity Cache (last level)
METRIC = "GEMM TFLOP/s at fp16 8192³ on 1 MI355X; % of dense MFMA peak"
HEADLINE = "nn_f16_8192"

# The configurations reported under "extra", each with its roofline (the 8192^3 bf16
# configuration first); the 256^3 one is a launch-latency case, not a roofline one.  The
# last is the matmul + ReLU epilogue after the Triton lecture notes (2048x2048x1024 fp16
# -> fp32; the notes give no size).
CONFIG_LINES = ["nn_bf16_8192", "tn_f16_8192", "tn_f16_256", "tn_f16_4096", "tn_f16_3000x5000x1000_f32out",
                "nn_bf16_3072x4096x4096_gelu", "nn_f16_2048x2048x1024_relu_f32out"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def warm_up(fn, launches, min_s, sync):
    """Run fn() at least `launches` times and for at least `min_s` seconds of back-to-back
    work (the GPU leaves its idle clock state over the first ~0.1-0.3 s); returns the
    launches and seconds actually run."""
    t0 = time.perf_counter()
    n = 0
    while n < launches:
        fn()
        n += 1
    sync()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            fn()
        n += 10
        sync()
    return n, time.perf_counter() - t0


def timed_launches(fn, steps, stream, sync):
    """Time `steps` launches back to back with HIP events recorded on the launch stream
    (torch's events wrap hipEventRecord).  The mean comes from one event pair around the
    whole window: an event recorded between two launches makes the second wait for the
    first to retire (measured ~6 us per launch on MI355X: 0 us gaps back to back, 5.6-6 us
    with an event after every launch), so no event sits inside it.  A second window of the
    same length, with an event every `block` launches, gives the median and the minimum of
    the block means (the event cost spread over the block)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sync()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    sync()
    wall = (time.perf_counter() - t0) / steps
    mean = e0.elapsed_time(e1) / steps
    block = max(1, min(10, steps // 4))
    nb = max(1, steps // block)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    ev[0].record(stream)
    for i in range(nb):
        for _ in range(block):
            fn()
        ev[i + 1].record(stream)
    sync()
    per = [ev[i].elapsed_time(ev[i + 1]) / block for i in range(nb)]
    return {"mean_ms": mean, "median_ms": statistics.median(per), "min_ms": min(per),
            "wall_ms": wall * 1e3, "block": block}


def graph_launches(fn, launches, replays, stream, sync):
    """For problems whose kernel is shorter than a host launch: `launches` calls captured
    in one HIP graph (gemm_run neither allocates nor synchronizes, so it captures), the
    graph replayed back to back between one event pair; returns the mean per launch."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(replays):
        e0.record()
        g.replay()
        e1.record()
        sync()
        per.append(e0.elapsed_time(e1) / launches)
    del g
    return {"mean_ms": statistics.mean(per), "median_ms": statistics.median(per), "min_ms": min(per),
            "wall_ms": None, "block": launches}


_inputs_cache = {}


def inputs_of(w):
    """Seeded inputs of workload w; the last workload's are kept (the ablation rows share
    theirs)."""
    import workloads as W
    key = (w.M, w.N, w.K, w.in_dtype, w.b_layout, w.dist)
    if key not in _inputs_cache:
        _inputs_cache.clear()
        _inputs_cache[key] = W.make_inputs(w)
    return _inputs_cache[key]


def time_gemm(w, steps, warmup, force=None, min_warmup_s=0.0, graph=False):
    """Times the GEMM of workload w (resident inputs); returns (timing dict, config).
    graph=True times launches captured in a HIP graph (for kernels shorter than a host
    launch)."""
    import numpy as np
    import torch

    import software_pipelined_tiled_gemm_amd as spg
    import workloads as W

    dev = torch.device("cuda:0")
    a, b = inputs_of(w)
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    B = torch.from_numpy(b.view(np.int16)).to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.int16 if w.out_dtype != W.F32 else torch.float32,
                    device=dev)
    stream = torch.cuda.current_stream(dev)
    sync = lambda: torch.cuda.synchronize(dev)
    g = spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue, force)
    cfg = g.config()
    run = lambda: g(A, B, C, stream)
    n_warm, s_warm = warm_up(run, warmup, min_warmup_s, sync)
    if graph:
        cur = lambda: g(A, B, C, torch.cuda.current_stream(dev))
        t = graph_launches(cur, 100, max(3, steps // 20), stream, sync)
    else:
        t = timed_launches(run, steps, stream, sync)
    t.update(warmup_launches_run=n_warm, warmup_s=round(s_warm, 3))
    g.close()
    del A, B, C
    torch.cuda.empty_cache()
    return t, cfg


def cold_line(w, launches=20):
    """The GEMM with cold caches: before each launch a 512 MiB write evicts the L2s and the
    256 MB Infinity Cache, so A and B come from HBM; one event pair around each launch
    (after its eviction write).  A context line next to the warm-cache figures."""
    import numpy as np
    import torch

    import software_pipelined_tiled_gemm_amd as spg
    import workloads as W

    dev = torch.device("cuda:0")
    a, b = inputs_of(w)
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    B = torch.from_numpy(b.view(np.int16)).to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.int16 if w.out_dtype != W.F32 else torch.float32,
                    device=dev)
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    per = []
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue) as g:
        g(A, B, C, stream)
        for i in range(launches + 2):
            evict.fill_(i & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g(A, B, C, stream)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            if i >= 2:
                per.append(e0.elapsed_time(e1) * 1e3)
    del A, B, C, evict
    torch.cuda.empty_cache()
    mean = statistics.mean(per)
    tf = w.flops / (mean * 1e-6) / 1e12
    return {"kernel_us_mean": round(mean, 2), "kernel_us_median": round(statistics.median(per), 2),
            "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_TFLOPS[w.in_dtype], 4),
            "launches": launches,
            "note": "cold caches: a 512 MiB write before each launch evicts the L2s and the "
                    "Infinity Cache; one event pair around each launch (context, not the metric)"}


def gemm_line(w, t, cfg):
    """One configuration's line: times (window mean, per-launch median and minimum), TFLOP/s
    and its MFMA roofline."""
    import workloads as W

    tf = w.flops / (t["mean_ms"] * 1e-3) / 1e12
    algo = 2 * (w.M * w.K + w.K * w.N) + (4 if w.out_dtype == W.F32 else 2) * w.M * w.N
    return {"M": w.M, "N": w.N, "K": w.K, "in_dtype": w.in_dtype, "out_dtype": w.out_dtype,
            "b_layout": w.b_layout, "epilogue": w.epilogue,
            "kernel_us_mean": round(t["mean_ms"] * 1e3, 2),
            "kernel_us_median": round(t["median_ms"] * 1e3, 2),
            "kernel_us_min": round(t["min_ms"] * 1e3, 2),
            "warmup_launches_run": t.get("warmup_launches_run"),
            "tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_TFLOPS[w.in_dtype],
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS[w.in_dtype], 4),
                         "traffic": measured_traffic(w.name, cfg, w), "algorithmic_bytes": algo},
            "config": cfg.as_dict()}


def time_gelu(n, dtype, steps, warmup):
    """Per-launch timing of the standalone GELU over n resident elements."""
    import numpy as np
    import torch

    import software_pipelined_tiled_gemm_amd as spg
    import workloads as W

    dev = torch.device("cuda:0")
    x = W.make_matrix((n,), dtype, ("normal", 1.0), W.SEED_A)
    X = torch.from_numpy(x.view(np.int16)).to(dev)
    Y = torch.empty_like(X)
    stream = torch.cuda.current_stream(dev)
    sync = lambda: torch.cuda.synchronize(dev)
    run = lambda: spg.gelu_run(X, Y, n, dtype, stream)
    warm_up(run, warmup, 0.0, sync)
    t = timed_launches(run, steps, stream, sync)
    del X, Y
    torch.cuda.empty_cache()
    return t


def copy_rate(nbytes, steps, warmup):
    """GB/s (read + write) of a plain device-to-device copy of nbytes: what the memory
    system gives a streaming kernel of that size, beside the 8 TB/s published peak."""
    import torch

    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize(dev)
    rate = 2 * nbytes / (e0.elapsed_time(e1) / steps * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return rate


def gelu_lines(steps, warmup):
    """The standalone GELU on the XLA page's bf16 [6,512,4096] tensor, whose 50 MB of
    input and output stay in the 256 MB Infinity Cache across back-to-back launches (so
    its rate is not an HBM figure), and on a tensor 16 times larger (805 MB moved per
    launch, far beyond that cache: the HBM roofline); then the GELU'd GEMM of that shape
    fused (epilogue) against unfused (GEMM, then GELU)."""
    import workloads as W

    out = {}
    for name, n in (("gelu_bf16_6x512x4096", 6 * 512 * 4096),
                    ("gelu_bf16_16x6x512x4096", 16 * 6 * 512 * 4096)):
        t = time_gelu(n, "bf16", steps, warmup)
        moved = 2 * n * 2
        gbs = moved / (t["mean_ms"] * 1e-3) / 1e9
        resident = moved <= MALL_BYTES
        out[name] = {
            "elements": n, "kernel_us_mean": round(t["mean_ms"] * 1e3, 2),
            "kernel_us_median": round(t["median_ms"] * 1e3, 2), "GB_per_s": round(gbs, 1),
            "device_copy_same_bytes_GB_per_s": round(copy_rate(moved // 2, steps, warmup), 1),
            "working_set": ("in + out fit the 256 MB Infinity Cache: cache-resident, not an "
                            "HBM figure" if resident else "in + out exceed the 256 MB Infinity "
                            "Cache: streamed from HBM")}
        if not resident:
            out[name]["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": moved}
        log(f"  {name}: {out[name]}")
    wf = W.WORKLOADS["nn_bf16_3072x4096x4096_gelu"]
    wp = W.custom(wf.M, wf.N, wf.K, wf.in_dtype, wf.out_dtype, wf.b_layout, "none", wf.dist,
                  name="nn_bf16_3072x4096x4096")
    t_fused, _ = time_gemm(wf, steps, warmup)
    t_plain, _ = time_gemm(wp, steps, warmup)
    t_gelu = time_gelu(wf.M * wf.N, "bf16", steps, warmup)
    k_f, k_p, k_g = t_fused["mean_ms"], t_plain["mean_ms"], t_gelu["mean_ms"]
    out["gemm_gelu_3072x4096x4096"] = {
        "fused_us": round(k_f * 1e3, 2), "gemm_us": round(k_p * 1e3, 2),
        "gelu_us": round(k_g * 1e3, 2), "unfused_us": round((k_p + k_g) * 1e3, 2),
        "fused_tflops": round(wf.flops / (k_f * 1e-3) / 1e12, 2)}
    return out


def cliff_line(steps, warmup):
    """K % 8 != 0 against its K % 8 == 0 neighbour (3000x5000x1001 / x1000, fp16, B [N,K],
    fp32 output): rows of A and B that are not 16-byte aligned."""
    import workloads as W

    base = W.WORKLOADS["tn_f16_3000x5000x1000_f32out"]
    odd = W.custom(base.M, base.N, 1001, base.in_dtype, base.out_dtype, base.b_layout,
                   base.epilogue, base.dist, name="tn_f16_3000x5000x1001_f32out")
    t_odd, cfg_odd = time_gemm(odd, steps, warmup)
    t_base, _ = time_gemm(base, steps, warmup)
    return {"K": 1001, "kernel_us_mean": round(t_odd["mean_ms"] * 1e3, 2),
            "tflops": round(odd.flops / (t_odd["mean_ms"] * 1e-3) / 1e12, 2),
            "neighbour_K1000_us_mean": round(t_base["mean_ms"] * 1e3, 2),
            "time_ratio_to_neighbour": round(t_odd["mean_ms"] / t_base["mean_ms"], 3),
            "config": cfg_odd.as_dict()}


def _socket_power_w():
    """Socket power the SMU reports (amd-smi metric -p), or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p"], capture_output=True, text=True, timeout=10)
        m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
        return float(m.group(1)) if m else None
    except Exception:
        return None


def _power_cap_w():
    """The package power limit (rocm-smi --showmaxpower), or None."""
    import json as _json
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower", "--json"], capture_output=True, text=True,
                           timeout=10)
        for card in _json.loads(r.stdout).values():
            v = card.get("Max Graphics Package Power (W)")
            if v is not None:
                return float(v)
    except Exception:
        pass
    return None


def sustained_clock(w, seconds=3.0):
    """Runs the workload back to back for `seconds` while sampling the engine clock
    (rocm-smi) and the socket power (amd-smi) the SMU reports; returns (median MHz,
    kernel us over the run, median socket W or None) or None."""
    import json as _json
    import subprocess
    import threading

    import numpy as np
    import torch

    import software_pipelined_tiled_gemm_amd as spg
    import workloads as W

    dev = torch.device("cuda:0")
    a, b = W.make_inputs(w)
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    B = torch.from_numpy(b.view(np.int16)).to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.int16 if w.out_dtype != W.F32 else torch.float32,
                    device=dev)
    samples, watts, stop = [], [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                                   text=True, timeout=10)
                for card in _json.loads(r.stdout).values():
                    v = str(card.get("sclk clock speed:", ""))
                    if "Mhz" in v:
                        samples.append(float(v.strip("()Mhz")))
            except Exception:
                return
            p = _socket_power_w()
            if p is not None:
                watts.append(p)
            time.sleep(0.2)

    g = spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue)
    for _ in range(10):
        g(A, B, C)
    torch.cuda.synchronize(dev)
    th = threading.Thread(target=sample)
    th.start()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0, n = time.time(), 0
    e0.record()
    while time.time() - t0 < seconds:
        for _ in range(25):
            g(A, B, C)
        n += 25
        torch.cuda.synchronize(dev)
    e1.record()
    torch.cuda.synchronize(dev)
    stop.set()
    th.join()
    g.close()
    del A, B, C
    torch.cuda.empty_cache()
    us = e0.elapsed_time(e1) * 1e3 / n
    if len(samples) < 3:
        return None
    samples = sorted(samples[1:])
    watts = sorted(watts[1:])
    return samples[len(samples) // 2], us, (watts[len(watts) // 2] if watts else None)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s=15.0):
    """The oracle (fp64 triple loop, OpenMP over rows), untuned, on a bounded sample of
    rows of the workload, sized for about target_s seconds."""
    import numpy as np

    import oracle
    import workloads as W

    a, b = W.make_inputs(w)
    o = oracle.default()
    nt = max(1, o.num_threads())

    def run(nrows):
        sel = np.linspace(0, w.M - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        o.gemm(a, b, w.M, w.N, w.K, w.in_dtype, w.b_layout, w.epilogue, rows=sel)
        return time.perf_counter() - t0

    # two-point calibration separates the fixed cost (decoding B) from the per-row cost
    r1, r2 = min(nt, w.M), min(4 * nt, w.M)
    t1 = run(r1)
    t2 = run(r2) if r2 > r1 else t1
    per_row = max((t2 - t1) / (r2 - r1), 1e-6) if r2 > r1 else max(t1 / r1, 1e-6)
    rows = int(min(w.M, max(r2, (target_s - t1 + r1 * per_row) / per_row)))
    rows = max(min(nt, w.M), rows - rows % nt if rows >= nt else rows)
    dt = run(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": o.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{rows} of {w.M} rows of C (all {w.N} columns, K={w.K}), {dt:.1f} s "
                      f"(B decoded once per call, included)"}


KERNEL_SOURCE = os.path.join(ROOT, "software_pipelined_tiled_gemm_amd", "csrc", "gemm_kernels.hpp")


def kernel_source_hash() -> str:
    """sha256 of the device code (the same recipe the counter summaries record)."""
    import hashlib

    with open(KERNEL_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def kernel_name(w, cfg) -> str:
    """The template instantiation a configuration launches (as profilers print it)."""
    b = lambda v: "true" if v else "false"
    # the persistent instantiation runs only on the shapes it takes (else its twin)
    pers = (cfg.persistent and not cfg.store and w.out_dtype != "f32" and w.K % cfg.block_k == 0
            and (w.b_layout == "nk" or w.N % cfg.block_n == 0))
    return (f"spg::pipelined_gemm<{b(w.in_dtype == 'bf16')}, {b(w.b_layout == 'nk')}, "
            f"{cfg.block_m}, {cfg.block_n}, {cfg.block_k}, {cfg.wave_m}, {cfg.wave_n}, "
            f"{cfg.stages}, {b(cfg.swizzle)}, {cfg.staging}, {cfg.lookahead}, {cfg.schedule}, "
            f"{b(pers)}, {cfg.mfma or 32}>")


def measured_traffic(workload: str, cfg, w):
    """HBM-side bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None unless it was taken on the same device code and the same kernel
    instantiation this run launches."""
    path = os.path.join(ROOT, "profiles", f"pipelined_gemm_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    src, traffic, kern = None, None, None
    for line in open(path):
        if "kernel sources sha256" in line:
            src = line.rsplit(":", 1)[1].strip()
        if "traffic_bytes_per_launch:" in line:
            traffic = float(line.split(":", 1)[1].strip())
        if line.startswith("# kernel:"):
            kern = line.split(":", 1)[1].strip()
    if src != kernel_source_hash() or kern is None or kernel_name(w, cfg) not in kern:
        return None
    return traffic


def parse_tile(spec):
    """'256x256x64:2[:swizzle[:group_m[:staging[:WMxWN[:lookahead[:schedule[:persistent[:store[:xcd_remap[:mfma]]]]]]]]]]'
    -> the matching
    compiled configuration (the first one in the table when the wave tile is not given)."""
    import software_pipelined_tiled_gemm_amd as spg

    parts = spec.split(":")
    dims = [int(x) for x in parts[0].lower().split("x")]
    bm, bn = dims[0], dims[1]
    bk = dims[2] if len(dims) > 2 else 64
    st = int(parts[1])
    swz = int(parts[2]) if len(parts) > 2 else 1
    gm = int(parts[3]) if len(parts) > 3 else 0
    stg = int(parts[4]) if len(parts) > 4 else 0
    wave = tuple(int(x) for x in parts[5].lower().split("x")) if len(parts) > 5 else None
    look = int(parts[6]) if len(parts) > 6 else 1
    sched = int(parts[7]) if len(parts) > 7 else 0
    pers = int(parts[8]) if len(parts) > 8 else 0
    store = int(parts[9]) if len(parts) > 9 else 0
    xcd = int(parts[10]) if len(parts) > 10 else 1
    mfma = int(parts[11]) if len(parts) > 11 else 32
    for i in range(spg.gemm_num_configs()):
        c = spg.gemm_list_config(i)
        if wave is not None and (c.wave_m, c.wave_n) != wave:
            continue
        if c.lookahead != look or c.schedule != sched or c.persistent != pers or c.mfma != mfma:
            continue
        if (c.block_m, c.block_n, c.block_k, c.stages, c.swizzle, c.staging) == (bm, bn, bk, st, swz, stg):
            if gm:
                c.group_m = gm
            c.store = store
            c.xcd_remap = xcd
            return c
    raise SystemExit(f"no compiled configuration matches --tile {spec}")


# Design-choice ablations at the headline workload: (label, --tile spec).  Each is a
# distinct kernel instantiation, so a profiler run over `--ablations` attributes
# counters to the rows by kernel name.
ABLATIONS = [
    ("default: 256x256x64, 8 waves of 128x64, 16x16x32 MFMAs, B one slot deeper than A (staging 6), compiler-placed schedule, group_m 4", "256x256x64:2:1:4:6:128x64:1:1:0:0:1:16"),
    ("the same with group_m 8 (the 32x32x16 kernel's best)", "256x256x64:2:1:8:6:128x64:1:1:0:0:1:16"),
    ("the same ring under the ping-pong schedule (the two waves of a SIMD take turns; the default for B stored [N,K])", "256x256x64:2:1:4:6:128x64:1:2:0:0:1:16"),
    ("two-slot ring (S=2), hand-placed schedule: the base of the 16x16x32 rows below", "256x256x64:2:1:4:0:128x64:1:0:0:0:1:16"),
    ("16x16x32, no swizzle", "256x256x64:2:0:4:0:128x64:1:0:0:0:1:16"),
    ("16x16x32, no overlap (S=1, the serial loop)", "256x256x64:1:1:4:0:128x64:1:0:0:0:1:16"),
    ("16x16x32, compiler-placed schedule", "256x256x64:2:1:4:0:128x64:1:1:0:0:1:16"),
    ("16x16x32, epilogue stored from registers (no LDS staging)", "256x256x64:2:1:4:0:128x64:1:0:0:1:1:16"),
    ("16x16x32, no tile remap (row-major raster, no XCD ranges)", "256x256x64:2:1:1:0:128x64:1:0:0:0:0:16"),
    ("16x16x32, 256x128 tile, 8 waves of 64x64, S=3", "256x128x64:3:1:4:0:64x64:1:0:0:0:1:16"),
    ("32x32x16 MFMAs (same tile)", "256x256x64:2:1:8:0:128x64:1:0"),
    ("32x32x16, A one slot deeper than B (staging 4)", "256x256x64:2:1:8:4:128x64:1:0"),
    ("no overlap (S=1, the serial loop), 4 waves", "256x256x64:1:1:8:0:128x128:1:0"),
    ("4 waves of 128x128 (one per SIMD), lookahead 1", "256x256x64:2:1:8:0:128x128:1:0"),
    ("4 waves of 128x128, lookahead 2", "256x256x64:2:1:8:0:128x128:2:0"),
    ("register-staged copies (VGPR -> ds_write), 8 waves", "256x256x64:2:1:8:1:128x64:1:0"),
    ("register-staged copies at any 2-byte alignment (staging 7, the misaligned-operand mode), 8 waves", "256x256x64:2:1:8:7:128x64:1:0"),
    ("copies spread over the barrier window (BK=32, S=5), 8 waves", "256x256x32:5:1:8:2:128x64:1:0"),
    ("compiler-placed schedule, 8 waves", "256x256x64:2:1:8:0:128x64:1:1"),
    ("swizzled LDS, BK=32, S=4, 4 waves", "256x256x32:4:1:8:0:128x128:1:0"),
    ("no swizzle, BK=32, S=4, 4 waves", "256x256x32:4:0:8:0:128x128:1:0"),
    ("256x128 tile, 8 waves of 64x64, S=3", "256x128x64:3:1:8:0:64x64:1:0"),
    ("256x128 tile, wave-specialized (producer wave + 4 consumers)", "256x128x64:3:1:8:3:128x64:1:0"),
    ("128x128 tile, 4 waves of 64x64, S=3", "128x128x64:3:1:8:0:64x64:1:0"),
    ("persistent: one workgroup per CU, its tiles as one k-tile stream", "256x256x64:2:1:8:0:128x64:1:0:1"),
    ("epilogue stored from registers (no LDS staging)", "256x256x64:2:1:8:4:128x64:1:0:0:1"),
    ("no tile remap (row-major raster, no XCD ranges)", "256x256x64:2:1:1:4:128x64:1:0:0:0:0"),
    ("XCD ranges only (group_m 1)", "256x256x64:2:1:1:4:128x64:1:0:0:0:1"),
    ("raster groups only (group_m 8, no XCD ranges)", "256x256x64:2:1:8:4:128x64:1:0:0:0:0"),
    ("128x128 tile, 4 waves of 64x64, S=2", "128x128x64:2:1:8:0:64x64:1:0"),
    ("128x128 tile, 4 waves of 64x64, S=4", "128x128x64:4:1:8:0:64x64:1:0"),
    ("128x128 tile, S=3, release delay 1 (S-1 in flight)", "128x128x64:3:1:8:5:64x64:1:0"),
    ("256x128 tile, 8 waves of 64x64, S=3, release delay 1", "256x128x64:3:1:8:5:64x64:1:0"),
]

# The tile-shape choice at the fused-GELU workload (3072x4096x4096, bf16 NN): how many
# tiles each shape makes against the 256 CUs.
GELU_ABLATIONS = [
    ("default: 192x256x64, S=2, 8 waves of 96x64, 16x16x32 (256 tiles: one per CU)", "192x256x64:2:1:4:0:96x64:1:0:0:0:1:16"),
    ("256x256x64, S=2, 8 waves of 128x64, 16x16x32 (192 tiles: 64 CUs idle)", "256x256x64:2:1:4:0:128x64:1:0:0:0:1:16"),
    ("256x256x64, 32x32x16 (192 tiles)", "256x256x64:2:1:4:0:128x64:1:0"),
    ("256x128x64, S=3, 8 waves of 64x64, 16x16x32 (384 tiles: 1.5 rounds)", "256x128x64:3:1:4:0:64x64:1:0:0:0:1:16"),
    ("128x128x64, S=3, 4 waves of 64x64, 32x32x16 (768 tiles: 3 rounds)", "128x128x64:3:1:4:0:64x64:1:0"),
    ("128x128x64, S=2, 8 waves of 32x64, 16x16x32 (768 tiles: 3 rounds)", "128x128x64:2:1:4:0:32x64:1:0:0:0:1:16"),
]

# The small-problem tile at the matmul + ReLU workload (2048x2048x1024 -> fp32): one round
# of 256 tiles of 128x128, or fewer, larger tiles
RELU_ABLATIONS = [
    ("default: 128x128x64, S=3, 8 waves of 32x64, 16x16x32 (256 tiles; 96 KiB: one workgroup per CU)", "128x128x64:3:1:4:0:32x64:1:0:0:0:1:16"),
    ("the same with S=2 (64 KiB: two workgroups can share a CU)", "128x128x64:2:1:4:0:32x64:1:0:0:0:1:16"),
    ("128x128x64, S=3, 4 waves of 64x64, 32x32x16 (the previous small-problem tile)", "128x128x64:3:1:4:0:64x64:1:0"),
    ("128x128x64, S=2, 4 waves of 64x64, 32x32x16", "128x128x64:2:1:4:0:64x64:1:0"),
    ("256x128x64, S=3, 8 waves of 64x64, 16x16x32, compiler-placed (128 tiles)", "256x128x64:3:1:4:0:64x64:1:1:0:0:1:16"),
    ("256x256x64, S=2, 8 waves of 128x64, 16x16x32 (64 tiles)", "256x256x64:2:1:4:0:128x64:1:0:0:0:1:16"),
]

ABLATIONS_BY_WORKLOAD = {"nn_bf16_3072x4096x4096_gelu": GELU_ABLATIONS,
                         "nn_f16_2048x2048x1024_relu_f32out": RELU_ABLATIONS}


def ablations_for(workload):
    """The ablation rows of a workload (the design-choice list unless it has its own)."""
    return ABLATIONS_BY_WORKLOAD.get(workload, ABLATIONS)


def run_ablations(w, steps, warmup, min_warmup_s):
    rows = []
    for label, spec in ablations_for(w.name):
        cfg = parse_tile(spec)
        # every row gets the same warm-up as the benchmark lines (at least min_warmup_s of
        # back-to-back launches, out of the clock ramp); kernels shorter than a host launch
        # are timed as launches captured in a HIP graph
        t, used = time_gemm(w, steps, warmup, cfg, min_warmup_s, graph=w.flops < 2e10)
        k = t["mean_ms"]
        rows.append({"label": label, "tile": spec, "kernel_us": round(k * 1e3, 2),
                     "kernel_us_median": round(t["median_ms"] * 1e3, 2),
                     "tflops": round(w.flops / (k * 1e-3) / 1e12, 2)})
        log(f"  {label}: {rows[-1]['kernel_us']} us, {rows[-1]['tflops']} TFLOP/s")
    print(json.dumps({"ablations": rows, "workload": w.name, "steps": steps, "warmup": warmup}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    # the GPU leaves its idle clock state over the first ~0.1-0.3 s of work: the warm-up
    # runs at least this long whatever --warmup says (the launches run are reported)
    ap.add_argument("--min-warmup-s", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=HEADLINE, help="workload name from workloads.WORKLOADS")
    ap.add_argument("--tile", default=None,
                    help="force a configuration: BMxBNxBK:S[:swizzle[:group_m[:staging[:WMxWN[:lookahead[:schedule[:persistent[:store[:xcd_remap[:mfma]]]]]]]]]] "
                         "(default: the library's choice)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra lines (every other configuration, the 8-GPU shard, the "
                         "K % 8 != 0 neighbour, the standalone GELU, fused vs unfused GELU GEMM, "
                         "the sustained clock)")
    ap.add_argument("--ablations", action="store_true",
                    help="time the design-choice ablations on the workload instead of the "
                         "benchmark line (ABLATIONS, or the workload's own list in "
                         "ABLATIONS_BY_WORKLOAD)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy 5 times, so that HBM "
                         "byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GEMM is "
              f"sharded across GPUs by rows of A with B replicated, which is not built here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = W.WORKLOADS[args.workload]
    log(f"bench: {w.describe()}")
    if args.ablations:
        run_ablations(w, args.steps, args.warmup, args.min_warmup_s)
        return
    force = parse_tile(args.tile) if args.tile else None
    t, cfg = time_gemm(w, args.steps, args.warmup, force, args.min_warmup_s)
    head = gemm_line(w, t, cfg)
    tflops = head["tflops"]
    log(f"  {cfg}: kernel {head['kernel_us_mean']} us mean, {head['kernel_us_median']} median, "
        f"{head['kernel_us_min']} min ({tflops} TFLOP/s); warm-up {t['warmup_launches_run']} "
        f"launches in {t['warmup_s']} s")

    extra = {}
    if args.workload == HEADLINE and not args.no_extra:
        steps = max(args.steps, 50)
        for name in CONFIG_LINES:
            wc = W.WORKLOADS[name]
            small = wc.flops < 1e9
            # kernels of ~20 us or less (under 20 GFLOP) run faster than the host can launch
            # them one by one: those are timed as launches captured in a HIP graph
            graph = wc.flops < 2e10
            tc, cc = time_gemm(wc, 200 if graph else steps, args.warmup, None,
                               0.2 if small else args.min_warmup_s, graph=graph)
            extra[name] = gemm_line(wc, tc, cc)
            if graph and not small:
                extra[name]["timing"] = ("100 launches captured in a HIP graph and replayed "
                                         "(the kernel is shorter than a host launch)")
            if small:
                extra[name]["note"] = ("4 tiles on 256 CUs: latency bound, the roofline fraction "
                                       "is not meaningful here; timed as 100 launches captured "
                                       "in a HIP graph (a host launch takes longer than the kernel)")
            if not args.no_cpu_baseline:
                extra[name]["cpu_baseline"] = cpu_baseline(wc, 2.0 if name != "nn_bf16_8192" else 6.0)
            log(f"  {name}: {extra[name]}")
        # one GPU's share of the 8-GPU row split (A and C by rows, B replicated)
        src = W.WORKLOADS["nn_bf16_8192"]
        wsh = W.custom(src.M // 8, src.N, src.K, src.in_dtype, src.out_dtype, src.b_layout,
                       src.epilogue, src.dist, name="nn_bf16_8192_shard_of_8")
        tsh, csh = time_gemm(wsh, steps, args.warmup)
        extra[wsh.name] = gemm_line(wsh, tsh, csh)
        log(f"  shard of 8: {extra[wsh.name]}")
        extra[f"{HEADLINE}_cold_caches"] = cold_line(W.WORKLOADS[HEADLINE])
        log(f"  cold caches: {extra[f'{HEADLINE}_cold_caches']}")
        extra["k_not_multiple_of_8"] = cliff_line(steps, args.warmup)
        log(f"  K % 8 != 0: {extra['k_not_multiple_of_8']}")
        extra.update(gelu_lines(steps, min(args.warmup, 200)))
        log(f"  fused vs unfused GELU GEMM: {extra['gemm_gelu_3072x4096x4096']}")
        for name in (HEADLINE, "nn_bf16_8192"):
            wc = W.WORKLOADS[name]
            clk = sustained_clock(wc)
            if clk is not None:
                mhz, us, watts = clk
                tf = wc.flops / (us * 1e-6) / 1e12
                extra[f"sustained_clock_{name}"] = {
                    "sclk_mhz_median": mhz, "kernel_us": round(us, 2), "tflops": round(tf, 2),
                    "frac_of_peak": round(tf / PEAK_TFLOPS[wc.in_dtype], 4),
                    "mfma_busy_at_that_clock": round(tf / (PEAK_TFLOPS[wc.in_dtype] * mhz / 2400.0), 4),
                    "socket_power_w_median": watts, "package_power_cap_w": _power_cap_w(),
                    "note": "3 s back-to-back run; clock (rocm-smi) and socket power (amd-smi) "
                            "sampled while it runs; peak scales with clock"}
                log(f"  sustained {name}: {extra[f'sustained_clock_{name}']}")

    if args.copy_calibration:
        src_t = torch.empty(128 << 20, dtype=torch.int16, device="cuda:0").fill_(1)
        dst_t = torch.empty_like(src_t)
        for _ in range(5):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        log("  copy calibration: 5 x 256 MiB read + 256 MiB written")
        del src_t, dst_t

    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches_run": t["warmup_launches_run"],
        "warmup_s": t["warmup_s"],
        "ms_per_step": round(t["mean_ms"], 4),
        "kernel_us_median": head["kernel_us_median"],
        "kernel_us_min": head["kernel_us_min"],
        "median_min_over": f"means of blocks of {t['block']} launches (one event per block)",
        "wall_ms_per_step": round(t["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "in_dtype": w.in_dtype,
                   "out_dtype": w.out_dtype, "b_layout": w.b_layout, "epilogue": w.epilogue,
                   "inputs": list(w.dist), "tile": cfg.as_dict(), "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS[w.in_dtype], 2),
        "roofline": head["roofline"],
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, 12.0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
