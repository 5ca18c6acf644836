"""The measurement contract of bench.py, checked on the CPU (no kernel runs): the shape
of a configuration line and its roofline, the link between a line's HBM-side traffic and
the committed rocprofv3 counter summaries, and the single-GPU guard."""

import os
import subprocess
import sys

import pytest

import software_pipelined_tiled_gemm_amd as spg
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    if not os.path.exists(spg.LIB_PATH):
        pytest.fail("libspgemm.so is not built; run __graft_entry__.build()")
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def _planned(w):
    h = spg.gemm_create(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue)
    try:
        return spg.gemm_get_config(h)
    finally:
        spg.gemm_destroy(h)


def _recorded(workload):
    """(kernel sources sha256, kernel name, traffic) a counter summary records, or None."""
    path = os.path.join(ROOT, "profiles", f"pipelined_gemm_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    src = kern = traffic = None
    for line in open(path):
        if "kernel sources sha256" in line:
            src = line.rsplit(":", 1)[1].strip()
        if line.startswith("# kernel:"):
            kern = line.split(":", 1)[1].strip()
        if "traffic_bytes_per_launch:" in line:
            traffic = float(line.split(":", 1)[1])
    return src, kern, traffic


def test_headline_is_the_metric_workload(bench):
    w = W.WORKLOADS[bench.HEADLINE]
    assert (w.M, w.N, w.K, w.in_dtype) == (8192, 8192, 8192, W.F16)
    assert "fp16 8192" in bench.METRIC
    for name in bench.CONFIG_LINES:
        assert name in W.WORKLOADS and name != bench.HEADLINE


@pytest.mark.parametrize("name", ["nn_f16_8192", "nn_bf16_8192", "tn_f16_8192", "tn_f16_4096",
                                  "tn_f16_3000x5000x1000_f32out", "nn_bf16_3072x4096x4096_gelu",
                                  "nn_f16_2048x2048x1024_relu_f32out"])
def test_configuration_line_and_roofline(bench, name):
    w = W.WORKLOADS[name]
    cfg = _planned(w)
    t = {"mean_ms": 0.5, "median_ms": 0.51, "min_ms": 0.49, "warmup_launches_run": 600}
    line = bench.gemm_line(w, t, cfg)
    r = line["roofline"]
    assert set(r) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(w.flops / 0.5e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    out_bytes = 4 if w.out_dtype == W.F32 else 2
    assert r["algorithmic_bytes"] == 2 * (w.M * w.K + w.K * w.N) + out_bytes * w.M * w.N
    assert line["kernel_us_mean"] == 500.0 and line["config"] == cfg.as_dict()
    # traffic comes from the committed counter summary, and only while it was taken on the
    # same device code and the instantiation this line launches
    rec = _recorded(name)
    if rec is None:
        assert r["traffic"] is None
        return
    src, kern, traffic = rec
    same = src == bench.kernel_source_hash() and bench.kernel_name(w, cfg) in kern
    if same:
        assert r["traffic"] == traffic
        assert traffic >= r["algorithmic_bytes"]     # memory-side bytes cover the compulsory ones
    else:
        assert r["traffic"] is None


def test_traffic_is_withheld_for_another_instantiation(bench):
    w = W.WORKLOADS["nn_f16_8192"]
    cfg = _planned(w)
    other = spg.TileConfig.from_dict({**cfg.as_dict(), "staging": 0, "schedule": 0})
    assert bench.measured_traffic(w.name, other, w) is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
