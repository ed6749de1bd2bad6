"""Host-side logic of bench.py, on the CPU: algorithmic byte counts, the
refusal of more than one GPU, the trace summary's cold/warm split and the
source-hash guard on recorded profiler figures."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from post_processing_amd import workloads as wl  # noqa: E402


def _shape(name, src, dst, mode, batch=1):
    import numpy as np
    frames = np.zeros((batch, src[1], src[0], 3), dtype=np.uint8)
    return wl.Workload(name, src[0], src[1], dst[0], dst[1], mode, (0, 0, 0), (1, 1, 1), 114.0,
                       0, frames, None)


@pytest.mark.parametrize("name,src,dst,mode,batch,total", [
    ("c1", (64, 48), (32, 32), wl.RESIZE, 1, 9_216 + 12_288),
    ("c2", (1920, 1080), (224, 224), wl.RESIZE, 1, 2_580_480 + 602_112),
    ("c3", (1280, 720), (640, 640), wl.LETTERBOX, 1, 2_764_800 + 4_915_200),
    ("c4", (3840, 2160), (384, 384), wl.RESIZE, 1, 8_847_360 + 1_769_472),
    ("c5t", (1280, 720), (224, 224), wl.RESIZE, 64, 148_635_648),
])
def test_algorithmic_bytes(name, src, dst, mode, batch, total):
    assert bench.preprocess_bytes(_shape(name, src, dst, mode, batch))["total"] == total


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert out.returncode == 2 and "one GPU" in out.stderr


def test_trace_summary_splits_cold_and_warm(tmp_path):
    rows = [("q1", 0, 400_000, "cache_flush_kernel"), ("q1", 400_500, 425_500, "pre"),
            ("q1", 430_000, 453_000, "pre"), ("q1", 453_100, 476_100, "pre"),
            ("q1", 500_000, 900_000, "cache_flush_kernel"), ("q1", 900_400, 926_400, "pre")]
    p = tmp_path / "t_kernel_trace.csv"
    with open(p, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp,Queue_Id\n")
        for q, a, b, n in rows:
            kname = ("void ws::(anonymous namespace)::cache_flush_kernel(uint4*)" if n != "pre"
                     else "void ws::(anonymous namespace)::preprocess_gather_kernel<float>(x)")
            f.write(f"\"{kname}\",{a},{b},{q}\n")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--trace-summary",
                          str(p), "--last", "3"], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    d = json.loads(out.stdout)
    key = "ws::preprocess_gather_kernel<float>"
    cold = d["preprocess_after_flush"][key]
    warm = d["preprocess_other"][key]
    assert cold["calls"] == 2 and warm["calls"] == 2
    assert cold["median_us"] == 25.5 and warm["mean_us"] == 23.0
    last = d["last_3"][key]
    assert last["calls"] == 3 and last["max_us"] == 26.0 and last["min_us"] == 23.0
    assert last["period_mean_us"] == (900.4 - 430.0) / 2 and last["queues"] == 1
    assert last["gap_mean_us"] == round(((453.1 - 453.0) + (900.4 - 476.1)) / 2, 3)


def test_recorded_figures_need_matching_sources(monkeypatch):
    monkeypatch.setitem(bench.MEASURED, "preprocess",
                        {"sha256_prefix": "0" * 16, "profile": "x",
                         "w": {"cold_us": 1.0, "warm_us": 1.0, "traffic": 1}})
    assert bench.measured("preprocess", "w") is None
    monkeypatch.setitem(bench.MEASURED["preprocess"], "sha256_prefix",
                        bench.sources_sha("preprocess")[:16])
    assert bench.measured("preprocess", "w")["traffic"] == 1
