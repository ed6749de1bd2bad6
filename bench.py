"""Benchmark of the fixed-shape frame pipeline on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --campaign [--report FILE]

One step = one replay of a lane's graph between the lane's two GPU events,
driven by the native submit/wait loop; the inputs are resident (device
memory, or the mapped host slot for the host-input lanes) before the timed
region starts.  Prints ONE JSON line.

Workloads (synthetic, seeded; shapes of the pages' classifier and detector
inputs):
  c5t  64 frames 1280x720 -> 224x224 in one launch (preprocess only): the
       bandwidth workload and the default
  c1   64x48 -> 32x32 + Top-5 of 1000 with planted ties
  c2   1920x1080 RGB8 -> 224x224 ImageNet-normalised + Top-5 of 1000
  c3   1280x720 -> 640x640 letterbox (pad 114, /255) + Top-32 of 8400x80
  c4   3840x2160 -> 384x384 + Top-32 of 21843 with 1% duplicates
  c5l  8 lanes, one host thread each, 1920x1080 from mapped host memory, Top-10
  c3d  c3's lane plus in-graph detection decode + NMS over a synthetic
       8400-anchor, 80-class head (conf 0.25, IoU 0.45, at most 300 boxes)

Latency percentiles always come from at least 10,000 replays (the timed
steps when there are that many, else a separate run after them); the sample
count is in the line.  The roofline describes the preprocess kernel: its
algorithmic bytes over its duration with cold caches (a flush kernel over a
buffer larger than the last-level cache runs before each launch, on the
lane's stream, outside the HIP-event interval), beside the back-to-back
(warm) duration and the rocprofv3 kernel durations and byte counters
recorded for the same kernel sources.

--campaign runs every workload (W = 1,000 warm-up and R = 10,000 timed
replays) in three campaigns with the workload order rotated, each with a
direct-launch repeat at the same counts, and times the CPU oracle's
preprocess and Top-K separately per workload (median of 5 after 1 warm-up).

Completion signals are polled by default (--signals polled puts
HSA_ENABLE_INTERRUPT=0 in the environment before the HIP runtime starts):
with the runtime's interrupt-driven default, each hipGraphLaunch spends
~15-25 us of host time, which is most of a single frame's replay.  The
default line also carries the C1/C2 lanes in this mode and C2 in the
interrupt-driven mode (a child process) for comparison.  --launch-cost times
the launch path alone with empty kernels.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "post_processing_amd", "csrc")

HBM_PEAK_GBS = 8000.0
MIN_LATENCY_SAMPLES = 10_000
LATENCY = {"samples": MIN_LATENCY_SAMPLES}
ALL_CORES: set = set()         # every core this process may use, before any pinning
TRACE_LAST = {"n": 0}
FLUSH_BYTES = 1 << 30          # > 256 MiB last-level cache (Infinity Cache)

# Sources each kernel compiles from: a recorded measurement is valid only
# while the sha256 of their concatenation is unchanged.
KERNEL_SOURCES = {
    "preprocess": ("ws_preprocess.hip", "ws_kernels.h"),
    "topk": ("ws_topk.hip", "ws_kernels.h", "ws_lanes.h"),
    "detect": ("ws_detect.hip", "ws_detect.h", "ws_lanes.h"),
}

# rocprofv3 measurements of the preprocess kernel, per workload (profiles/
# holds the summaries and the commands).  `cold_us` / `warm_us`: median
# kernel duration from --kernel-trace of `bench.py` itself, for the launches
# that follow a cache flush and for the back-to-back ones (`bench.py
# --trace-summary` splits the trace).  `traffic`: HBM bytes per launch from
# two --pmc passes (FETCH_SIZE, then WRITE_SIZE), scaled by what the same
# counters read for a plain 256 MiB device copy.
MEASURED = {
    "preprocess": {
        "sha256_prefix": "bb32d75899624327",
        "profile": "profiles/preprocess_c5t_64x1280x720_to_224.md",
        # The 64-frame batch runs the gather kernel with the streaming cache
        # policy (non-temporal frame loads and tensor stores).  cold: the 400
        # launches rotated over four lanes' batches, start-to-start period
        # (kernel median 25.237 us); warm: the median of the other launches
        # of this grid (back-to-back stage launches and graph replays).
        # traffic: FETCH_SIZE 53,799.5 KiB x 2.0 + WRITE_SIZE 37,632 KiB per
        # launch (median of 547 dispatches), calibrated on a 256 MiB device
        # copy (FETCH_SIZE 131,083.5 KiB, WRITE_SIZE 262,144 KiB).
        "c5t_64x1280x720_to_224": {"cold_us": 25.305, "cold_kernel_us": 25.237,
                                   "warm_us": 22.317, "traffic": 110_181_376 + 38_535_168},
    },
}


def sources_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured(kernel: str, workload: str):
    """The recorded rocprofv3 figures for this kernel and workload, or None
    when the kernel's sources have changed since they were taken."""
    m = MEASURED.get(kernel, {})
    if not m.get("sha256_prefix") or sources_sha(kernel)[:16] != m["sha256_prefix"]:
        return None
    rec = m.get(workload)
    return dict(rec, profile=m["profile"]) if rec else None


# ---------------------------------------------------------------------------
# Algorithmic bytes (what the method must move at minimum, per launch).

def touched_rows(src: int, dst: int) -> int:
    rows = set()
    for d in range(dst):
        num = max((2 * d + 1) * src - dst, 0)
        i0 = num // (2 * dst)
        rows.add(i0)
        rows.add(min(i0 + 1, src - 1))
    return len(rows)


def region(w) -> tuple[int, int]:
    """(region_w, region_h) of the resampled area inside the tensor."""
    if w.mode == 0:
        return w.dst_w, w.dst_h
    from fractions import Fraction
    r = min(Fraction(w.dst_w, w.src_w), Fraction(w.dst_h, w.src_h))
    rw = max(1, min(w.dst_w, int(w.src_w * r + Fraction(1, 2))))
    rh = max(1, min(w.dst_h, int(w.src_h * r + Fraction(1, 2))))
    return rw, rh


TENSOR = {"dtype": "f32"}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def preprocess_bytes(w) -> dict:
    """Source rows the taps touch (read whole) + the tensor, per launch."""
    rw, rh = region(w)
    src = touched_rows(w.src_h, rh) * 3 * w.src_w * w.batch
    out = 3 * w.dst_w * w.dst_h * ELEM_BYTES[TENSOR["dtype"]] * w.batch
    return {"read": src, "write": out, "total": src + out}


def topk_bytes(w) -> int:
    return 0 if not w.k else 4 * w.num_scores + 8 * w.k


def detect_bytes(w, candidates: int, kept: int) -> int:
    """Decode reads every anchor's class probabilities and each candidate's
    64 box logits, and writes a 16-byte box, an 8-byte key and a 2-byte place
    in its class per candidate, a count per 64 anchors and the per-class
    counts; suppression reads those back (clearing the class counts) and
    writes 24 bytes per kept box plus the 8-byte header."""
    nc, a = w.det["nc"], w.head.shape[1]
    groups = (a + 63) // 64
    return (4 * nc * a + candidates * (256 + 2 * (16 + 8 + 2)) + 24 * kept + 8
            + 8 * groups + 12 * nc)


# ---------------------------------------------------------------------------

def pct(a, q):
    return float(np.percentile(a, q))


def lat_stats(ms: np.ndarray) -> dict:
    us = np.asarray(ms, dtype=np.float64) * 1e3
    n = int(us.size)
    p99 = pct(us, 99) if n >= 1000 else None
    return {"samples": n, "p50_us": pct(us, 50), "p99_us": p99, "mean_us": float(us.mean()),
            "max_us": float(us.max()), "min_us": float(us.min()),
            "p99_over_p50": (p99 / pct(us, 50)) if p99 is not None else None}


KNOBS = {}
INPUT_OVERRIDE = {}


def make_lane(w, torch, host_input=None, use_graph=True):
    from post_processing_amd import ws
    host = w.host_input if host_input is None else host_input
    mode = INPUT_OVERRIDE.get("mode")
    if mode is None:
        mode = ws.INPUT_MAPPED_HOST if host else ws.INPUT_DEVICE
    host = mode != ws.INPUT_DEVICE
    dev = torch.device("cuda:0")
    keep = {}
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[TENSOR["dtype"]]
    keep["tensor"] = torch.empty((w.batch, 3, w.dst_h, w.dst_w), dtype=tdt, device=dev)
    if w.k:
        keep["scores"] = torch.from_numpy(w.scores).to(dev)
    if not host:
        keep["frames"] = torch.from_numpy(np.ascontiguousarray(w.frames)).to(dev)
    det = {}
    if w.head is not None:
        keep["head"] = torch.from_numpy(np.ascontiguousarray(w.head)).to(dev)
        det = dict(det_classes=w.det["nc"], det_max_det=w.det["max_det"], det_conf=w.det["conf"],
                   det_iou=w.det["iou"], det_agnostic=w.det["agnostic"],
                   det_head_dev=keep["head"])
    torch.cuda.synchronize()
    cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h,
                         batch=w.batch, letterbox=(w.mode == 1), pad=w.pad, mean=w.mean,
                         std=w.std, num_scores=w.num_scores, k=w.k, input_mode=mode,
                         use_graph=use_graph, input_dev=keep.get("frames"),
                         scores_dev=keep.get("scores"), tensor_dev=keep["tensor"],
                         tensor_dtype={"f32": ws.DTYPE_F32, "f16": ws.DTYPE_F16,
                                       "bf16": ws.DTYPE_BF16}[TENSOR["dtype"]], **det, **KNOBS)
    lane = ws.Lane(cfg)
    if host:
        lane.input_host_array()[...] = w.frames
    lane._keep = keep
    return lane


def stage_times(lane, w, launches: int) -> dict:
    """Per-kernel mean duration from back-to-back launches between HIP events
    on the lane's stream (warm caches), and the algorithmic bandwidth."""
    from post_processing_amd import ws
    pb = preprocess_bytes(w)
    out = {}
    ms = lane.time_stage(ws.STAGE_PREPROCESS, launches)
    out["preprocess"] = {"us": ms * 1e3, "bytes": pb["total"], "gbs": pb["total"] / (ms * 1e-3) / 1e9}
    if w.k:
        ms = lane.time_stage(ws.STAGE_TOPK, launches)
        tb = topk_bytes(w)
        out["topk"] = {"us": ms * 1e3, "bytes": tb, "gbs": tb / (ms * 1e-3) / 1e9}
    if w.head is not None:
        ms = lane.time_stage(ws.STAGE_DETECT, launches)
        _, scores, _, cand = lane.detections()
        db = detect_bytes(w, cand, len(scores))
        out["detect"] = {"us": ms * 1e3, "bytes": db, "gbs": db / (ms * 1e-3) / 1e9,
                         "candidates": cand, "kept": len(scores)}
    return out


def topk_marks(lane, reps: int = 30) -> dict:
    """Phase times of the Top-K kernels from the clock-mark build
    (libws_marks.so): one Top-K launch at a time, its marks read back; the
    median over `reps` launches of each phase, in microseconds (100 MHz
    clock, 0.01 us resolution)."""
    import ctypes
    from post_processing_amd import ws
    lib = ws.load()
    fn = lib.ws_debug_topk_marks
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32]
    fn.restype = ctypes.c_int
    plan = lane.plan()
    G, W = plan["topk_groups"], plan["topk_block"] // 64
    merge0 = 1 << 16
    n = merge0 + 64
    buf = np.zeros(n, dtype=np.uint64)
    rows = []
    for _ in range(reps):
        fn(None, 0, 1)
        lane.time_stage(ws.STAGE_TOPK, 1)
        fn(buf.ctypes.data, n, 0)
        m = buf[:G * 4 * 8].reshape(G, 4, 8)[:, :W, :].astype(np.int64)
        t0 = m[:, :, 0].min()
        us = lambda a: float(a) * 0.01   # noqa: E731
        r = {"partial_wave_start_spread": us(m[:, :, 0].max() - t0),
             "partial_load": us(np.median(m[:, :, 1] - m[:, :, 0])),
             "partial_select": us(np.median(m[:, :, 2] - m[:, :, 1])),
             "select_threshold": us(np.median(m[:, :, 5] - m[:, :, 1])),
             "select_screen_compact": us(np.median(m[:, :, 6] - m[:, :, 5])),
             "select_merge_survivors": us(np.median(m[:, :, 7] - m[:, :, 6])),
             "partial_block_merge": us(np.median(m[:, 0, 3] - m[:, 0, 2])),
             "partial_publish": us(np.median(m[:, 0, 4] - m[:, 0, 3])),
             "partial_span": us(m[:, 0, 4].max() - t0)}
        if G > 1:
            f = buf[merge0:merge0 + 32].reshape(4, 8)[:, :5].astype(np.int64)
            if (f[:, 0] > 0).all():
                r.update({"merge_start_after_partials": us(f[:, 0].min() - m[:, 0, 4].max()),
                          "merge_load": us(np.median(f[:, 1] - f[:, 0])),
                          "merge_fold": us(np.median(f[:, 2] - f[:, 1])),
                          "merge_block_merge": us(f[0, 3] - f[0, 2]),
                          "merge_write": us(f[0, 4] - f[0, 3]),
                          "total_span": us(f[0, 4] - t0)})
        rows.append(r)
    keys = rows[0].keys()
    return {k: round(float(np.median([r[k] for r in rows if k in r])), 3) for k in keys}


def detect_marks(lane, reps: int = 30) -> dict:
    """Phase times of the detection kernels from the clock-mark build
    (libws_marks.so): one detection launch (decode + suppression) at a time,
    its marks read back; the median over `reps` launches of each phase, in
    microseconds (100 MHz clock)."""
    import ctypes
    from post_processing_amd import ws
    lib = ws.load()
    fn = lib.ws_debug_detect_marks
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32]
    fn.restype = ctypes.c_int
    nms0 = 1 << 16
    prof0 = nms0 + 4096
    n = prof0 + 16 * 8
    buf = np.zeros(n, dtype=np.uint64)
    rows = []
    us = lambda a: float(a) * 0.01   # noqa: E731
    for _ in range(reps):
        fn(None, 0, 1)
        lane.time_stage(ws.STAGE_DETECT, 1)
        fn(buf.ctypes.data, n, 0)
        d = buf[:nms0].reshape(-1, 8).astype(np.int64)
        d = d[d[:, 0] > 0]
        t = buf[nms0:nms0 + 256].reshape(16, 16).astype(np.int64)
        live = t[:, 0] > 0
        t = t[live]
        pf = buf[prof0:prof0 + 128].reshape(16, 8).astype(np.int64)[live]
        t0 = d[:, 0].min()
        full = d[d[:, 5] > 0]
        r = {"decode_waves": int(d.shape[0]),
             "decode_start_spread": us(d[:, 0].max() - t0),
             "decode_class_scan": us(np.median(d[:, 1] - d[:, 0])),
             "decode_compact": us(np.median(d[:, 2] - d[:, 1])),
             "decode_dfl": us(np.median(full[:, 3] - full[:, 2])) if len(full) else 0.0,
             "decode_sync": us(np.median(full[:, 4] - full[:, 3])) if len(full) else 0.0,
             "decode_store": us(np.median(full[:, 5] - full[:, 4])) if len(full) else 0.0,
             "decode_span": us(d[:, 1:6].max() - t0),
             "nms_start_after_decode": us(t[:, 0].min() - d[:, 1:6].max()),
             "nms_counts_starts_runs": us(t[0, 1] - t[0, 0]),
             "nms_clear_and_wide_scan": us(t[0, 12] - t[0, 1]),
             "nms_gather": us(t[0, 11] - t[0, 12]),
             "nms_gather_barrier": us(t[0, 2] - t[0, 11]),
             "nms_order": us(t[0, 3] - t[0, 2]),
             "nms_sort_all": us(t[0, 4] - t[0, 3]),
             "nms_runs_busiest": us(t[:, 5].max() - t[0, 4]),
             "nms_runs_median_wave": us(np.median(t[:, 5] - t[:, 4])),
             "nms_runs_barrier": us(t[0, 6] - t[:, 5].max()),
             "nms_kept_rank": us(t[0, 7] - t[0, 6]),
             "nms_output": us(t[0, 8] - t[0, 7]),
             "nms_span": us(t[0, 8] - t[:, 0].min()),
             "runs_per_wave_max": int(t[:, 9].max()),
             "cycles_busiest_wave": {k: int(pf[int(np.argmax(t[:, 5])), i]) for i, k in enumerate(
                 ("loads", "screen", "settle", "screen_steps", "kept", "blocks", "round_waits",
                  "w0_round_screen"))},
             "cycles_wave0": {k: int(pf[0, i]) for i, k in enumerate(
                 ("loads", "screen", "settle", "screen_steps", "kept", "blocks", "round_waits",
                  "w0_round_screen"))},
             "total_span": us(t[0, 8] - t0)}
        rows.append(r)
    out = {}
    for k in rows[0].keys():
        if isinstance(rows[0][k], dict):
            out[k] = {j: int(np.median([r[k][j] for r in rows])) for j in rows[0][k]}
        else:
            out[k] = round(float(np.median([r[k] for r in rows])), 3)
    return out


def cold_times(lane, torch, launches: int = 20) -> dict:
    """Preprocess launches each after a flush kernel on the lane's stream
    (HIP events around the launch only, so each interval also holds one
    dispatch and the events' own overhead): a 1 GiB read flush, a 2 GiB read
    flush (if the first evicts everything, doubling it changes nothing) and
    a 1 GiB write flush (whose dirty lines the timed launch writes back).
    Medians in microseconds."""
    from post_processing_amd import ws
    buf = torch.ones((2 * FLUSH_BYTES) // 4, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    out = {}
    for name, nbytes, write in (("flush_read_1GiB", FLUSH_BYTES, False),
                                ("flush_read_2GiB", 2 * FLUSH_BYTES, False),
                                ("flush_write_1GiB", FLUSH_BYTES, True)):
        ms = lane.time_stage_cold(ws.STAGE_PREPROCESS, buf, nbytes, launches, write=write)
        out[name] = float(np.median(ms)) * 1e3
    del buf
    torch.cuda.empty_cache()
    return out


ROTATE_LANES = 4          # 3 x 148.6 MB touched between a batch's turns: > 256 MiB
ROTATE_LAUNCHES = 400


def rotated_times(w, torch, lane0) -> dict:
    """Preprocess launches back to back over several lanes' buffers in turn
    (HIP events around the whole run on the first lane's stream): with 4
    lanes of the 64-frame batch, 446 MB pass through the caches between two
    turns of a batch, so each launch reads its frames from HBM.  2 and 6
    lanes bracket it (2 leaves part of the batch cached; 6 must match 4 if 4
    already evicts everything).  The 4-lane run goes last, so its launches
    are the last ones of this grid in a profiler trace.  Microseconds per
    launch."""
    from post_processing_amd import ws
    lanes = [lane0] + [make_lane(w, torch) for _ in range(5)]
    try:
        out = {}
        for n in (2, 6, ROTATE_LANES):
            out[f"rotate_{n}_lanes"] = ws.time_stage_rotate(
                lanes[:n], ws.STAGE_PREPROCESS, ROTATE_LAUNCHES, warmup=2 * n) * 1e3
    finally:
        for ln in lanes[1:]:
            ln.destroy()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def rotation_probe(torch, launches: int = 400) -> int:
    """Which costs a rotated launch pays: 400 preprocess launches of the
    64-frame batch back to back over four lanes in turn, with the lanes'
    inputs and tensors shared or distinct.  Prints one JSON line
    (microseconds per launch, three repeats each)."""
    from post_processing_amd import workloads as wl
    from post_processing_amd import ws
    w = wl.c5_throughput(64)
    dev = torch.device("cuda:0")
    frames = [torch.from_numpy(w.frames).to(dev) for _ in range(4)]
    tensors = [torch.empty((64, 3, 224, 224), dtype=torch.float32, device=dev) for _ in range(4)]
    torch.cuda.synchronize()

    def lane(fi, ti):
        cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h,
                             batch=w.batch, mean=w.mean, std=w.std, input_mode=ws.INPUT_DEVICE,
                             input_dev=frames[fi], tensor_dev=tensors[ti])
        return ws.Lane(cfg)

    cases = {"shared_inputs_shared_tensors": [(0, 0)] * 4,
             "shared_inputs_distinct_tensors": [(0, i) for i in range(4)],
             "distinct_inputs_shared_tensors": [(i, 0) for i in range(4)],
             "distinct_inputs_distinct_tensors": [(i, i) for i in range(4)]}
    out = {"metric": "preprocess us per launch, 400 launches rotated over 4 lanes",
           "workload": w.name}
    for name, pairs in cases.items():
        lanes = [lane(f, t) for f, t in pairs]
        ws.time_stage_rotate(lanes, ws.STAGE_PREPROCESS, 40, warmup=8)
        out[name] = [round(ws.time_stage_rotate(lanes, ws.STAGE_PREPROCESS, launches,
                                                warmup=8) * 1e3, 3) for _ in range(3)]
        for ln in lanes:
            ln.destroy()
    print(json.dumps(out), flush=True)
    return 0


def roofline_obj(w, stages: dict, cold: dict | None) -> dict:
    """The preprocess kernel against HBM: the stage that moves the frame and
    the tensor, and the one the metric names.  Top-K (a few KB to 2.7 MB)
    and detection are latency-bound chains of one or a few workgroups, which
    a bandwidth roofline does not describe; their times are in `kernels`."""
    pb = preprocess_bytes(w)["total"]
    warm_us = stages["preprocess"]["us"]
    key = f"rotate_{ROTATE_LANES}_lanes"
    us = cold[key] if cold and key in cold else warm_us
    gbs = pb / (us * 1e-6) / 1e9
    rec = measured("preprocess", w.name)
    out = {"kernel": "preprocess", "bound": "hbm", "achieved": round(gbs, 2),
           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5),
           "traffic": rec["traffic"] if rec else None,
           "bytes_per_launch": pb, "us_per_launch": round(us, 3),
           "caches": (f"cold: {ROTATE_LAUNCHES} launches back to back over {ROTATE_LANES} "
                      f"lanes' buffers in turn" if cold else "warm: back to back on one lane"),
           "warm": {"us_per_launch": round(warm_us, 3),
                    "frac": round(pb / (warm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)},
           "profiled": None}
    if cold:
        out["cold_checks_us"] = {k: round(v, 3) for k, v in cold.items() if k != key}
    if rec:
        prof = {"profile": rec["profile"], "cold_period_us": rec["cold_us"],
                "cold_kernel_us": rec["cold_kernel_us"], "warm_kernel_us": rec["warm_us"],
                "cold_frac": round(pb / (rec["cold_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)}
        prof["live_over_profiled"] = round(us / rec["cold_us"], 4) if cold else None
        out["profiled"] = prof
    slow = max(stages, key=lambda s: stages[s]["us"])
    out["slowest_stage"] = {"kernel": slow, "us_per_launch": round(stages[slow]["us"], 3)}
    return out


def run_replays(lane, torch, steps: int, warmup: int) -> dict:
    """Warm-up, then `steps` timed replays (the timed region), then -- when
    fewer than MIN_LATENCY_SAMPLES were timed -- more replays for the
    latency percentiles."""
    lane.bench(warmup)
    torch.cuda.synchronize()
    ms, wall, host_us, sub_us = lane.bench(steps, host=True)
    torch.cuda.synchronize()
    res = {"frames_per_s": steps * lane.cfg.batch / wall, "wall_s": wall}
    if steps < LATENCY["samples"]:
        ms, _, host_us, sub_us = lane.bench(LATENCY["samples"], host=True)
        torch.cuda.synchronize()
        res["latency_source"] = f"{LATENCY['samples']} replays after the timed steps"
    else:
        res["latency_source"] = "the timed steps"
    res.update(lat_stats(ms))
    wait_us = host_us - sub_us
    res["host"] = {"p50_us": pct(host_us, 50), "p99_us": pct(host_us, 99),
                   "submit_p50_us": pct(sub_us, 50), "submit_p99_us": pct(sub_us, 99),
                   "wait_p50_us": pct(wait_us, 50), "wait_p99_us": pct(wait_us, 99)}
    return res


def run_lanes(lanes, torch, steps: int, warmup: int) -> dict:
    from post_processing_amd import ws
    ws.bench_lanes(lanes, warmup)
    torch.cuda.synchronize()
    ms, wall = ws.bench_lanes(lanes, steps)
    torch.cuda.synchronize()
    res = {"frames_per_s": len(lanes) * lanes[0].cfg.batch * steps / wall, "wall_s": wall,
           "per_lane_p50_us": [pct(m * 1e3, 50) for m in ms]}
    if len(lanes) * steps < LATENCY["samples"]:
        ms, _ = ws.bench_lanes(lanes, -(-LATENCY["samples"] // len(lanes)))
        torch.cuda.synchronize()
    res.update(lat_stats(ms.ravel()))
    return res


def pinned_h2d_gbs(torch, nbytes: int = 64 << 20, reps: int = 20) -> float:
    """Host-to-device copy rate from pinned host memory (one DMA copy of
    `nbytes`, `reps` times, between HIP events): the PCIe reference beside the
    kernel's own mapped-read rate."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        d.copy_(h, non_blocking=True)
    e1.record()
    e1.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del h, d
    return gbs


def cache_keep_figures(w, torch) -> dict:
    """The C5T preprocess with ordinary (cached) frame loads and tensor stores
    (WS_CACHE_KEEP) beside the streaming default: warm (the same batch back to
    back, so it is read from the last-level cache) and cold (rotated over four
    lanes' batches), in microseconds per launch."""
    from post_processing_amd import ws
    held = KNOBS.get("cache_policy")
    KNOBS["cache_policy"] = ws.CACHE_KEEP
    try:
        lane = make_lane(w, torch)
        try:
            warm = lane.time_stage(ws.STAGE_PREPROCESS, 500) * 1e3
            cold = rotated_times(w, torch, lane)[f"rotate_{ROTATE_LANES}_lanes"]
        finally:
            lane.destroy()
    finally:
        KNOBS["cache_policy"] = held
    b = preprocess_bytes(w)["total"]
    return {"warm_us": round(warm, 3), "warm_frac": round(b / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
            "cold_us": round(cold, 3), "cold_frac": round(b / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)}


def c5l_figures(torch, steps: int = 1000, warmup: int = 100) -> dict:
    """C5L beside the default line: eight lanes reading 1920x1080 frames from
    mapped host memory, one host thread each; the preprocess kernel's
    mapped-read rate; the pinned-host DMA copy rate on the same box."""
    from post_processing_amd import workloads as wl
    from post_processing_amd import ws
    work = [wl.c5_lane(i) for i in range(8)]
    lanes = [make_lane(x, torch) for x in work]
    # Lane threads inherit this thread's affinity: let them spread over every
    # core this process may use (all eight on the one pinned core drop the
    # rate by a quarter and add a multi-millisecond tail), then pin back.
    held = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if held is not None:
        os.sched_setaffinity(0, ALL_CORES or held)
    try:
        res = run_lanes(lanes, torch, steps, warmup)
        us = lanes[0].time_stage(ws.STAGE_PREPROCESS, 200) * 1e3
        read = preprocess_bytes(work[0])["read"]
        out = {"lanes": 8, "frames_per_s": round(res["frames_per_s"], 1),
               "p50_us": round(res["p50_us"], 3),
               "p99_us": round(res["p99_us"], 3) if res["p99_us"] else None,
               "latency_samples": res["samples"], "preprocess_us": round(us, 3),
               "mapped_host_read_gbs": round(read / (us * 1e-6) / 1e9, 2),
               "pinned_h2d_copy_gbs": round(pinned_h2d_gbs(torch), 2),
               "transfers_included": True}
    finally:
        if held is not None:
            os.sched_setaffinity(0, held)
        for ln in lanes:
            ln.destroy()
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, one thread, on the host of this run.

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def oracle_stage_times(w, reps: int = 5) -> dict:
    """O-PRE and O-TOPK (and the detection oracle when the workload has a
    head) timed separately on one thread: the median of `reps` calls after
    one warm-up call each, in milliseconds."""
    from threadpoolctl import threadpool_limits

    from oracle import letterbox_region, preprocess_batch, topk
    from oracle import detect as odet
    stages = {"o_pre": lambda: preprocess_batch(w.frames, w.dst_w, w.dst_h, w.mean, w.std,
                                                letterbox=(w.mode == 1), pad=w.pad)}
    if w.k:
        stages["o_topk"] = lambda: topk(w.scores, w.k)
    if w.head is not None:
        reg = (letterbox_region(w.src_w, w.src_h, w.dst_w, w.dst_h) if w.mode == 1
               else (0, 0, w.dst_w, w.dst_h))
        stages["o_detect"] = lambda: odet.detect(w.head, w.src_w, w.src_h, w.dst_w, w.dst_h, reg,
                                                 w.det["nc"], w.det["conf"], w.det["iou"],
                                                 w.det["max_det"], w.det["agnostic"])
    out = {}
    with threadpool_limits(1):
        for name, fn in stages.items():
            fn()
            t = []
            for _ in range(reps):
                t0 = time.perf_counter()
                fn()
                t.append(time.perf_counter() - t0)
            out[name + "_ms"] = float(np.median(t)) * 1e3
    return out


def cpu_baseline(w) -> dict:
    st = oracle_stage_times(w)
    per_frame_ms = sum(st.values()) / w.batch
    stages = " + ".join(k[:-3].replace("o_", "O-").upper() for k in st)
    return {"value": round(1e3 / per_frame_ms, 3), "unit": "frames/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{w.name}: {stages} timed separately, median of 5 calls after 1 "
                       f"warm-up each, {w.batch} frame{'s' if w.batch > 1 else ''} per call, "
                       f"1 thread; value = frames / sum of the stage medians"),
            "stages_ms": {k: round(v, 3) for k, v in st.items()},
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


_POOL = {}


def _pool_init(cores, frames: int) -> None:
    os.sched_setaffinity(0, cores)
    from threadpoolctl import threadpool_limits
    from post_processing_amd import workloads as wl
    _POOL["limit"] = threadpool_limits(1)
    _POOL["w"] = wl.c5_throughput(frames)


def _pool_frame(i: int) -> float:
    from oracle import preprocess_batch
    w = _POOL["w"]
    out = preprocess_batch(w.frames[i:i + 1], w.dst_w, w.dst_h, w.mean, w.std,
                           letterbox=(w.mode == 1), pad=w.pad)
    return float(out[0, 0, 0, 0])


def cpu_baseline_pool(w, cores, budget_s: float = 10.0) -> dict:
    """The same oracle over a process pool, one frame per task and one thread
    per worker, for the batched workload: whole passes over the batch until
    the budget is spent."""
    import multiprocessing as mp
    n = max(1, min(16, len(cores)))
    ctx = mp.get_context("spawn")     # children start clean and never touch the GPU
    with ctx.Pool(n, initializer=_pool_init, initargs=(set(cores), w.batch)) as pool:
        # Each pass is bounded: a pool whose workers die at start-up would
        # otherwise wait for them forever.
        pool.map_async(_pool_frame, range(w.batch), chunksize=1).get(timeout=300)   # warm-up
        passes = 0
        t0 = time.perf_counter()
        while passes < 2 or time.perf_counter() - t0 < budget_s:
            pool.map_async(_pool_frame, range(w.batch), chunksize=1).get(timeout=120)
            passes += 1
        dt = time.perf_counter() - t0
    return {"value": round(passes * w.batch / dt, 3), "unit": "frames/s", "cores": n,
            "kind": "oracle",
            "sample": f"{passes} passes over the {w.batch} frames of {w.name} (float64 "
                      f"preprocess), {n} worker processes, one frame per task, 1 thread each",
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


# ---------------------------------------------------------------------------
# Run record: versions, GPU state, PCIe link, inputs.

def under_profiler() -> bool:
    """True when a profiler's library is preloaded into this process: then
    every child process initialises the GPU before it runs, so the helpers
    below start no other program."""
    return ("rocprof" in os.environ.get("LD_PRELOAD", "")
            or any(k.startswith("ROCPROF") for k in os.environ))


def versions() -> dict:
    out = {"python": platform.python_version(), "numpy": np.__version__}
    try:
        import torch
        out["torch"] = torch.__version__
        out["hip"] = getattr(torch.version, "hip", None)
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            out["rocm"] = f.read().strip()
    except OSError:
        pass
    # The HIP runtime the lanes actually run on (the first one loaded wins).
    try:
        with open("/proc/self/maps") as f:
            out["hip_runtime_files"] = sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        pass
    return out


def _flatten(obj, prefix=""):
    if isinstance(obj, dict):
        for k, v in obj.items():
            yield from _flatten(v, f"{prefix}.{k}" if prefix else str(k))
    elif isinstance(obj, list):
        for i, v in enumerate(obj):
            yield from _flatten(v, f"{prefix}[{i}]")
    else:
        yield prefix, obj


def gpu_state() -> dict:
    """Clocks, power, temperature and PCIe link of GPU 0 from `amd-smi metric
    --json`: the graphics clock of every XCD, the memory clock, socket power,
    hotspot and memory temperatures, link width and speed."""
    if under_profiler():
        return {"tool": None, "skipped": "profiled run"}
    try:
        r = subprocess.run(["amd-smi", "metric", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:   # amd-smi absent or its output not JSON
        return {"tool": None, "error": str(e)[:200]}
    g = (data.get("gpu_data") or [data])[0] if isinstance(data, dict) else data[0]

    def val(*path):
        o = g
        for k in path:
            if not isinstance(o, dict) or k not in o:
                return None
            o = o[k]
        return o.get("value") if isinstance(o, dict) else (None if o == "N/A" else o)

    clocks = g.get("clock", {}) if isinstance(g, dict) else {}
    gfx = [val("clock", k, "clk") for k in sorted(clocks) if k.startswith("gfx_")]
    return {"tool": "amd-smi", "gfx_clk_mhz": gfx, "gfx_max_clk_mhz": val("clock", "gfx_0", "max_clk"),
            "mem_clk_mhz": val("clock", "mem_0", "clk"),
            "socket_power_w": val("power", "socket_power"),
            "hotspot_temp_c": val("temperature", "hotspot"),
            "mem_temp_c": val("temperature", "mem"),
            "pcie_width": val("pcie", "width"), "pcie_speed_gts": val("pcie", "speed")}


def pcie_link() -> dict:
    """PCIe link of the GPU(s) from sysfs (current and maximum speed and
    width), plus amd-smi's bus report when available."""
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        rec = {}
        for name in ("current_link_speed", "current_link_width", "max_link_speed",
                     "max_link_width"):
            try:
                with open(os.path.join(dev, name)) as f:
                    rec[name] = f.read().strip()
            except OSError:
                pass
        if rec:
            out[os.path.basename(os.path.dirname(dev))] = rec
    if under_profiler():
        return out
    try:
        r = subprocess.run(["amd-smi", "static", "--bus", "--json"], capture_output=True,
                           text=True, timeout=30)
        if r.returncode == 0 and r.stdout.strip():
            try:
                flat = dict(_flatten(json.loads(r.stdout)))
                out["amd_smi_bus"] = {k: v for k, v in flat.items()
                                      if any(s in k.lower() for s in ("pcie", "link", "width",
                                                                      "speed", "bdf"))}
            except ValueError:
                out["amd_smi_bus"] = r.stdout[:1000]
    except Exception:
        pass
    return out


def input_hashes(w) -> dict:
    from post_processing_amd import workloads as wl
    out = {"frames": wl.sha256(w.frames)}
    if w.k:
        out["scores"] = wl.sha256(w.scores)
    if w.head is not None:
        out["head"] = wl.sha256(w.head)
    return out


def copy_calibration(torch, args) -> int:
    """A plain device-to-device copy of known size, the reference for scaling
    the profiler's byte counters (FETCH_SIZE / WRITE_SIZE) to real bytes."""
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    for _ in range(args.warmup if args.warmup < 10 else 3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"metric": "device copy bandwidth (calibration)", "value": 2 * n / dt / 1e9,
                      "unit": "GB/s", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "steps": args.steps}), flush=True)
    return 0


SIGNALS = {"mode": None}


def apply_signals(requested: str) -> str:
    """Put the signal-wait mode in the environment before the HIP runtime
    starts and return the mode in effect.  With the runtime's default
    interrupt-driven signals every hipGraphLaunch spent ~15-25 us of host time
    on this system; polled signals (HSA_ENABLE_INTERRUPT=0) take that to
    ~2-4 us (`--launch-cost`).  Under a profiler the runtime is already up, so
    the shell's setting is what holds."""
    if under_profiler():
        mode = "polled" if os.environ.get("HSA_ENABLE_INTERRUPT") == "0" else "interrupt"
        if mode != requested:
            print(f"bench.py: under a profiler the HIP runtime started before this script; "
                  f"signals stay {mode} (set HSA_ENABLE_INTERRUPT in the shell)", file=sys.stderr)
        return mode
    if requested == "polled":
        os.environ["HSA_ENABLE_INTERRUPT"] = "0"
    else:
        os.environ.pop("HSA_ENABLE_INTERRUPT", None)
    return requested


def single_frame_figures(torch, names=("c1", "c2")) -> dict:
    """Single-frame lanes beside the default line: 1,000 warm-up and
    MIN_LATENCY_SAMPLES timed replays each, on this process's signal mode."""
    out = {}
    for name in names:
        w = load_workload(name)
        lane = make_lane(w, torch)
        try:
            res = run_replays(lane, torch, LATENCY["samples"], 1000)
        finally:
            lane.destroy()
        out[workload_name(name, w)] = {
            "frames_per_s": round(res["frames_per_s"], 1), "p50_us": round(res["p50_us"], 3),
            "p99_us": round(res["p99_us"], 3), "p99_over_p50": round(res["p99_over_p50"], 4),
            "latency_samples": res["samples"],
            "host_p50_us": round(res["host"]["p50_us"], 3),
            "host_p99_us": round(res["host"]["p99_us"], 3),
            "host_in_submit_p50_us": round(res["host"]["submit_p50_us"], 3)}
    return out


def interrupt_signal_figures(pinned) -> dict | None:
    """C2 with the runtime's interrupt-driven signals, in a child process (the
    mode is fixed when the HIP runtime starts): the comparison for the polled
    default."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "c2",
           "--signals", "interrupt", "--steps", str(LATENCY["samples"]), "--warmup", "1000",
           "--no-cpu-baseline", "--no-extras", "--no-direct"]
    if pinned is not None:
        cmd += ["--pin-core", str(pinned)]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=180)
    except subprocess.TimeoutExpired:
        return None
    if r.returncode != 0 or not r.stdout.strip():
        print(f"[bench] interrupt-signal comparison failed: {r.stderr[-400:]}", file=sys.stderr)
        return None
    d = json.loads(r.stdout.strip().splitlines()[-1])
    h = d.get("host_submit_to_return_us") or {}
    return {"workload": d["config"]["workload"], "signals": d["config"].get("signals"),
            "p50_us": d["p50_us"], "p99_us": d["p99_us"], "p99_over_p50": d["p99_over_p50"],
            "latency_samples": d["latency_samples"], "host_p50_us": h.get("p50"),
            "host_p99_us": h.get("p99"), "host_in_submit_p50_us": h.get("in_submit_p50")}


def launch_cost(args) -> int:
    """The launch path alone: empty kernels, 224 x 256 threads each."""
    from post_processing_amd import ws
    forms = {"graph": ws.LAUNCH_GRAPH, "direct": ws.LAUNCH_DIRECT}
    rows = []
    for nodes in (1, 2, 4):
        for fname, form in forms.items():
            r = ws.launch_cost(nodes, form, replays=3000, warmup=300)
            row = {"nodes": nodes, "form": fname}
            for key, arr in r.items():
                row[key + "_us"] = {q: round(pct(arr, v), 2)
                                    for q, v in (("p50", 50), ("p90", 90), ("p99", 99))}
                row[key + "_us"]["min"] = round(float(arr.min()), 2)
            rows.append(row)
            print(f"[launch-cost] {nodes} node(s) {fname}: launch {row['launch_us']['p50']} us, "
                  f"event interval {row['gpu_us']['p50']} us (p99 {row['gpu_us']['p99']})",
                  file=sys.stderr, flush=True)
    rec = {"metric": "launch path alone: host time of the launch call(s), host time to "
                     "completion observed, event interval; empty kernels",
           "signals": SIGNALS["mode"], "replays": 3000, "warmup": 300, "rows": rows,
           "versions": versions()}
    print(json.dumps(rec), flush=True)
    return 0


def load_workload(name: str):
    from post_processing_amd import workloads as wl
    if name == "c5l":
        return [wl.c5_lane(i) for i in range(8)]
    if name == "c5t":
        return wl.c5_throughput(64)
    if name == "c3d":
        return wl.c3d()
    if name in ("dense_any", "dense_class"):
        return wl.dense_detect(agnostic=name == "dense_any")
    return wl.ALL_CONFIGS[name]()


def workload_name(name: str, w) -> str:
    return "c5l_8lanes_1920x1080_to_224_mapped" if name == "c5l" else w.name


# ---------------------------------------------------------------------------
# Campaign: every workload, graph and direct launch, three rotated passes.

CAMPAIGN_ORDER = ["c1", "c2", "c3", "c4", "c5l", "c5t"]


def campaign(torch, args) -> int:
    warm, reps = args.campaign_warmup, args.campaign_replays
    works = {}
    for name in CAMPAIGN_ORDER:
        t0 = time.perf_counter()
        works[name] = load_workload(name)
        print(f"[campaign] inputs for {name} in {time.perf_counter() - t0:.1f} s",
              file=sys.stderr, flush=True)
    lanes = {}
    for name, w in works.items():
        for graph in (True, False):
            ws_list = w if name == "c5l" else [w]
            lanes[(name, graph)] = [make_lane(x, torch, use_graph=graph) for x in ws_list]
    runs = []
    for c in range(3):
        order = CAMPAIGN_ORDER[c:] + CAMPAIGN_ORDER[:c]
        for name in order:
            for graph in (True, False):
                ls = lanes[(name, graph)]
                if len(ls) > 1:
                    # One host thread per lane, spread over every core (the
                    # threads inherit this thread's affinity).
                    held = os.sched_getaffinity(0)
                    os.sched_setaffinity(0, ALL_CORES or held)
                    try:
                        res = run_lanes(ls, torch, reps, warm)
                    finally:
                        os.sched_setaffinity(0, held)
                else:
                    res = run_replays(ls[0], torch, reps, warm)
                runs.append({"campaign": c, "workload": name, "graph": graph,
                             **{k: (round(v, 3) if isinstance(v, float) else v)
                                for k, v in res.items()}})
                print(f"[campaign] {c} {name} graph={graph}: {res['frames_per_s']:.0f} frames/s,"
                      f" p50 {res['p50_us']:.2f} us, p99/p50 {res['p99_over_p50']:.3f}",
                      file=sys.stderr, flush=True)
    summary = {}
    for name in CAMPAIGN_ORDER:
        for graph in (True, False):
            rs = [r for r in runs if r["workload"] == name and r["graph"] == graph]
            summary[f"{name}_{'graph' if graph else 'direct'}"] = {
                "frames_per_s": [r["frames_per_s"] for r in rs],
                "p50_us": [r["p50_us"] for r in rs], "p99_us": [r["p99_us"] for r in rs],
                "p99_over_p50": [r["p99_over_p50"] for r in rs],
                "host_p50_us": [round(r["host"]["p50_us"], 3) for r in rs if "host" in r],
                "host_in_submit_p50_us": [round(r["host"]["submit_p50_us"], 3)
                                          for r in rs if "host" in r]}
    for ls in lanes.values():
        for ln in ls:
            ln.destroy()
    oracle = {}
    if not args.no_cpu_baseline:
        for name in CAMPAIGN_ORDER:
            w = works[name][0] if name == "c5l" else works[name]
            oracle[name] = {k: round(v, 3) for k, v in oracle_stage_times(w).items()}
            print(f"[campaign] oracle {name}: {oracle[name]}", file=sys.stderr, flush=True)
    rec = {"metric": "campaign: frames/s and p50/p99 us per graph replay, graph vs direct launch",
           "warmup_replays": warm, "timed_replays": reps, "campaigns": 3,
           "order": [CAMPAIGN_ORDER[c:] + CAMPAIGN_ORDER[:c] for c in range(3)],
           "signals": SIGNALS["mode"],
           "summary": summary, "oracle_ms_1_thread": oracle, "cpu": cpu_model(),
           "host_cpus": os.cpu_count(), "versions": versions(), "gpu_state": gpu_state(),
           "pcie": pcie_link(),
           "input_sha256": {n: (input_hashes(w[0]) if n == "c5l" else input_hashes(w))
                            for n, w in works.items()},
           "transfers_included": {"c5l": True, **{n: False for n in CAMPAIGN_ORDER if n != "c5l"}}}
    if args.report:
        with open(args.report, "w") as f:
            json.dump({**rec, "runs": runs}, f, indent=1)
    print(json.dumps(rec), flush=True)
    return 0


# ---------------------------------------------------------------------------

def trace_summary(path: str) -> int:
    """Summarise a rocprofv3 kernel trace (`*_kernel_trace.csv`) of this
    benchmark: per kernel and grid, the dispatch count and mean / median
    duration; for the preprocess kernel, separately the launches that
    directly follow a cache flush on the same queue and the others; with
    --last N, also the last N dispatches of each kernel and grid (the rotated
    cold launches, which bench.py runs last).  Runs on the CPU; prints JSON."""
    import csv
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    recs = []
    for r in rows:
        name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name") or ""
        t0 = int(r.get("Start_Timestamp") or r.get("BeginNs") or 0)
        t1 = int(r.get("End_Timestamp") or r.get("EndNs") or 0)
        q = r.get("Queue_Id") or r.get("Stream_Id") or "0"
        grid = r.get("Grid_Size") or r.get("Grid_Size_X") or ""
        if r.get("Grid_Size_Y") not in (None, "", "1"):
            grid = f"{grid}x{r['Grid_Size_Y']}"   # frames of a batch in y
        recs.append((q, t0, t1, name, grid))
    recs.sort(key=lambda x: (x[0], x[1]))
    by = {}
    spans = {}
    cold, warm = {}, {}
    prev = {}
    for q, t0, t1, name, grid in recs:
        us = (t1 - t0) * 1e-3
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        key = f"{short} grid={grid}" if grid else short
        by.setdefault(key, []).append(us)
        spans.setdefault(key, []).append((t0, t1, q))
        if "preprocess" in short:
            side = cold if "cache_flush_kernel" in prev.get(q, "") else warm
            side.setdefault(key, []).append(us)
        prev[q] = short

    if TRACE_LAST["n"]:
        # The last N dispatches (by start time) of each kernel and grid:
        # bench.py runs its rotated cold launches last among the preprocess
        # launches of a grid.
        last_spans = {k: sorted(v)[-TRACE_LAST["n"]:] for k, v in spans.items()}
        out_last = {k: [(b - a) * 1e-3 for a, b, _ in v] for k, v in last_spans.items()}
    else:
        out_last = None

    def stats(v):
        return {"calls": len(v), "mean_us": round(float(np.mean(v)), 3),
                "median_us": round(float(np.median(v)), 3), "min_us": round(float(np.min(v)), 3),
                "max_us": round(float(np.max(v)), 3)}

    out = {"trace": path, "kernels": {k: stats(v) for k, v in sorted(by.items())}}
    if out_last:
        last = {}
        for k, v in sorted(out_last.items()):
            rec = stats(v)
            sp = last_spans[k]
            rec["queues"] = len({q for _, _, q in sp})
            if len(sp) > 1:
                # Start-to-start period of consecutive dispatches (what a
                # back-to-back run's event time per launch measures) and the
                # idle time between one dispatch's end and the next's start.
                rec["period_mean_us"] = round((sp[-1][0] - sp[0][0]) * 1e-3 / (len(sp) - 1), 3)
                rec["gap_mean_us"] = round(float(np.mean([(b[0] - a[1]) * 1e-3
                                                          for a, b in zip(sp, sp[1:])])), 3)
            last[k] = rec
        out[f"last_{TRACE_LAST['n']}"] = last
    for label, side in (("preprocess_after_flush", cold), ("preprocess_other", warm)):
        if side:
            out[label] = {k: stats(v) for k, v in sorted(side.items())}
    print(json.dumps(out, indent=1))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="c5t",
                    choices=["c1", "c2", "c3", "c4", "c5l", "c5t", "c3d", "dense_any", "dense_class",
                             "copy"])
    ap.add_argument("--campaign", action="store_true",
                    help="every workload, three rotated campaigns, graph and direct launch")
    ap.add_argument("--campaign-warmup", type=int, default=1000)
    ap.add_argument("--campaign-replays", type=int, default=10000)
    ap.add_argument("--copy-mib", type=int, default=256,
                    help="copy workload: bytes per device-to-device copy (MiB)")
    ap.add_argument("--stage-launches", type=int, default=500)
    ap.add_argument("--cold-launches", type=int, default=20)
    ap.add_argument("--rows-per-group", type=int, default=0, help="preprocess tuning knob (0 = auto)")
    ap.add_argument("--topk-chunk", type=int, default=0, help="Top-K tuning knob (0 = auto)")
    ap.add_argument("--dtype", default="f32", choices=["f32", "f16", "bf16"],
                    help="tensor element type (arithmetic stays FP32)")
    ap.add_argument("--input", default=None, choices=["device", "mapped", "copy"],
                    help="override the workload's input mode")
    ap.add_argument("--pixels-per-thread", type=int, default=0,
                    help="preprocess tuning knob: 1, 2 or 4 (0 = auto)")
    ap.add_argument("--cache-policy", default="auto", choices=["auto", "keep", "stream"],
                    help="the preprocess kernel's frame loads and tensor stores (WS_CACHE_*)")
    ap.add_argument("--autotune", action="store_true",
                    help="let each lane time candidate launch geometries at create")
    ap.add_argument("--wait", default="spin", choices=["spin", "block"],
                    help="how ws_wait waits for the done event")
    ap.add_argument("--lanes", type=int, default=1,
                    help="lanes driven at once, one host thread each, each with its own "
                         "buffers (not c5l, which is eight lanes): one lane's work runs while "
                         "another's is launched")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-direct", action="store_true", help="skip the direct-launch comparison")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the C5L figures and the cold-cache launches")
    ap.add_argument("--report", default=None, help="also write a detailed JSON report here")
    ap.add_argument("--graph-packet-capture", choices=["off", "runtime-default"],
                    default="runtime-default",
                    help="HIP runtime graph mode (DEBUG_CLR_GRAPH_PACKET_CAPTURE), read once when "
                         "HIP starts; 'off' only for comparison")
    ap.add_argument("--pin-core", type=int, default=-2,
                    help="run the submit/wait loop on this host core (-2: the last core this "
                         "process may use; -1: no pinning); single-lane workloads only")
    ap.add_argument("--latency-samples", type=int, default=MIN_LATENCY_SAMPLES,
                    help="replays the latency percentiles are taken over, at least (lower it "
                         "only for profiler runs, where every dispatch is slowed)")
    ap.add_argument("--rotation-probe", action="store_true",
                    help="preprocess launches rotated over lanes with shared or distinct "
                         "inputs and tensors (which costs a cold launch pays)")
    ap.add_argument("--marks", action="store_true",
                    help="load the clock-mark build (libws_marks.so, built with `python -m "
                         "post_processing_amd.build --marks`) and add Top-K and detection "
                         "phase times")
    ap.add_argument("--trace-summary", default=None, metavar="CSV",
                    help="summarise a rocprofv3 kernel trace of this benchmark and exit (CPU)")
    ap.add_argument("--signals", default="polled", choices=["polled", "interrupt"],
                    help="how the HIP runtime waits for completion signals: polled "
                         "(HSA_ENABLE_INTERRUPT=0, set before HIP starts) or the runtime's "
                         "interrupt-driven default")
    ap.add_argument("--launch-cost", action="store_true",
                    help="time the launch path alone (empty kernels: graph replay against "
                         "direct launches) and print one JSON record")
    ap.add_argument("--last", type=int, default=0,
                    help="with --trace-summary: also summarise the last N dispatches of each "
                         "kernel and grid")
    args = ap.parse_args(argv)
    if args.trace_summary:
        TRACE_LAST["n"] = args.last
        return trace_summary(args.trace_summary)
    LATENCY["samples"] = args.latency_samples
    if args.graph_packet_capture == "off":
        # Must be in the environment before torch (or anything else) starts HIP.
        os.environ["DEBUG_CLR_GRAPH_PACKET_CAPTURE"] = "0"
    SIGNALS["mode"] = apply_signals(args.signals)
    pinned = None
    all_cores = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    ALL_CORES.update(all_cores)
    if args.pin_core != -1 and hasattr(os, "sched_setaffinity"):
        allowed = sorted(os.sched_getaffinity(0))
        pinned = allowed[-1] if args.pin_core == -2 else args.pin_core
        if pinned not in allowed:
            print(f"bench.py: core {pinned} is not available to this process", file=sys.stderr)
            return 2

    if args.gpus != 1:
        print(f"bench.py: this pipeline runs on one GPU per process; --gpus {args.gpus} is not "
              "supported (lanes and frames shard across GPUs with no exchange; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    from post_processing_amd import ws
    if args.marks:
        from post_processing_amd import build as ppbuild
        ws.load(ppbuild.LIB_MARKS)
    ws.load()

    KNOBS.update(rows_per_group=args.rows_per_group, topk_chunk=args.topk_chunk,
                 pixels_per_thread=args.pixels_per_thread, autotune=args.autotune,
                 cache_policy={"auto": ws.CACHE_AUTO, "keep": ws.CACHE_KEEP,
                               "stream": ws.CACHE_STREAM}[args.cache_policy],
                 wait_mode=ws.WAIT_BLOCK if args.wait == "block" else ws.WAIT_SPIN)
    TENSOR["dtype"] = args.dtype
    if args.input:
        INPUT_OVERRIDE["mode"] = {"device": ws.INPUT_DEVICE, "mapped": ws.INPUT_MAPPED_HOST,
                                  "copy": ws.INPUT_COPY}[args.input]
    if args.launch_cost:
        if pinned is not None:
            os.sched_setaffinity(0, {pinned})
        return launch_cost(args)
    if args.workload == "copy":
        return copy_calibration(torch, args)
    if args.rotation_probe:
        return rotation_probe(torch)
    if args.campaign:
        if pinned is not None:
            os.sched_setaffinity(0, {pinned})
        return campaign(torch, args)
    name = args.workload
    t_gen = time.perf_counter()
    loaded = load_workload(name)
    work = loaded if name == "c5l" else None
    w = loaded[0] if name == "c5l" else loaded
    print(f"[bench] inputs for {name} ready in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    extra = {}
    if args.lanes != 1 and (name == "c5l" or args.lanes < 1 or args.lanes > 8):
        print("bench.py: --lanes takes 1..8 (c5l is eight lanes by definition)", file=sys.stderr)
        return 2
    multi = name == "c5l" or args.lanes > 1
    if multi:
        # Several lanes, one host thread each: threads inherit the creator's
        # affinity, so pinning here would put them all on one core.
        pinned = None
    if pinned is not None:
        os.sched_setaffinity(0, {pinned})   # this thread runs every submit/wait loop below
    cold = None
    if multi:
        lanes = [make_lane(x, torch) for x in (work if name == "c5l" else [w] * args.lanes)]
        res = run_lanes(lanes, torch, args.steps, args.warmup)
        res["latency_source"] = "replays of all lanes"
        res["plan"] = lanes[0].plan()
        lane = lanes[0]
        stages = stage_times(lane, w, args.stage_launches)
        if name == "c5l":
            pb = preprocess_bytes(w)
            extra["mapped_host_read_gbs"] = pb["read"] / (stages["preprocess"]["us"] * 1e-6) / 1e9
            extra["pinned_h2d_copy_gbs"] = pinned_h2d_gbs(torch)
        steps_total = len(lanes) * args.steps
    else:
        lane = make_lane(w, torch)
        res = run_replays(lane, torch, args.steps, args.warmup)
        res["plan"] = lane.plan()
        stages = stage_times(lane, w, args.stage_launches)
        steps_total = args.steps
        if lane.cfg.input_mode != ws.INPUT_DEVICE:
            pb = preprocess_bytes(w)
            if lane.cfg.input_mode == ws.INPUT_MAPPED_HOST:
                extra["mapped_host_read_gbs"] = (pb["read"] / (stages["preprocess"]["us"] * 1e-6)
                                                 / 1e9)
            extra["pinned_h2d_copy_gbs"] = pinned_h2d_gbs(torch)
        if not args.no_direct:
            dl = make_lane(w, torch, use_graph=False)
            dres = run_replays(dl, torch, min(args.steps, LATENCY["samples"]),
                               min(args.warmup, 1000))
            extra["direct_launch"] = {"frames_per_s": round(dres["frames_per_s"], 1),
                                      "p50_us": round(dres["p50_us"], 3),
                                      "p99_us": round(dres["p99_us"], 3),
                                      "latency_samples": dres["samples"]}
            dl.destroy()
        if not args.no_extras and lane.cfg.input_mode == ws.INPUT_DEVICE:
            print("[bench] cold-cache launches", file=sys.stderr, flush=True)
            cold = cold_times(lane, torch, args.cold_launches)
            cold.update(rotated_times(w, torch, lane))
            extra["rotate_launches"] = ROTATE_LAUNCHES
        if name == "c5t" and not args.no_extras:
            print("[bench] C5L lanes", file=sys.stderr, flush=True)
            extra["c5l"] = c5l_figures(torch)
            if lane.plan().get("streaming"):
                print("[bench] the same batch with cached loads and stores", file=sys.stderr,
                      flush=True)
                extra["cache_keep"] = cache_keep_figures(w, torch)
            print("[bench] single-frame lanes", file=sys.stderr, flush=True)
            extra["single_frame"] = single_frame_figures(torch)
            if SIGNALS["mode"] == "polled" and not under_profiler():
                print("[bench] C2 with interrupt-driven signals (child process)",
                      file=sys.stderr, flush=True)
                torch.cuda.synchronize()
                extra["single_frame_interrupt_signals"] = interrupt_signal_figures(pinned)

    if args.marks and w.k:
        extra["topk_marks_us"] = topk_marks(lane)
    if args.marks and w.det:
        extra["detect_marks_us"] = detect_marks(lane)
    roof = roofline_obj(w, stages, cold)
    input_mode = args.input or ("mapped" if (w.host_input or name == "c5l") else "device")
    line = {
        "metric": "frames/s and p50/p99 us per graph replay; preprocess HBM GB/s vs peak",
        "value": round(res["frames_per_s"], 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": steps_total,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_s"] * 1e3 / steps_total, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.dtype == "f32" else f"f32->{args.dtype}",
        "data": "synthetic",
        "config": {"workload": workload_name(name, w),
                   "frames_per_step": w.batch, "src": [w.src_w, w.src_h],
                   "dst": [w.dst_w, w.dst_h], "letterbox": w.mode == 1,
                   "topk": {"n": w.num_scores, "k": w.k} if w.k else None,
                   "detect": ({"anchors": int(w.head.shape[1]), **{k: w.det[k] for k in
                              ("nc", "conf", "iou", "max_det")}} if w.head is not None else None),
                   "input": input_mode,
                   "graph": True, "lanes": 8 if name == "c5l" else args.lanes,
                   "wait": args.wait,
                   "signals": SIGNALS["mode"],
                   "cache_policy": "stream" if res["plan"].get("streaming") else "keep",
                   "graph_packet_capture": args.graph_packet_capture,
                   "host_core": pinned,
                   "parallelism": "single_gpu"},
        "p50_us": round(res["p50_us"], 3),
        "p99_us": round(res["p99_us"], 3) if res["p99_us"] is not None else None,
        "p99_over_p50": round(res["p99_over_p50"], 4) if res["p99_over_p50"] else None,
        "latency_samples": res["samples"],
        "latency_source": res["latency_source"],
        # Host view of the same replays: just before ws_submit to ws_wait's return.
        "host_submit_to_return_us": ({"p50": round(res["host"]["p50_us"], 3),
                                      "p99": round(res["host"]["p99_us"], 3),
                                      "in_submit_p50": round(res["host"]["submit_p50_us"], 3),
                                      "in_submit_p99": round(res["host"]["submit_p99_us"], 3),
                                      "in_wait_p50": round(res["host"]["wait_p50_us"], 3),
                                      "in_wait_p99": round(res["host"]["wait_p99_us"], 3)}
                                     if "host" in res else None),
        "transfers_included": input_mode != "device",
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in stages.items()},
        "plan": res["plan"],
        "roofline": roof,
    }
    line.update({k: (round(v, 3) if isinstance(v, float) else v) for k, v in extra.items()})
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
        if name == "c5t" and all_cores:
            print("[bench] timing the CPU oracle over a process pool", file=sys.stderr, flush=True)
            line["cpu_baseline_pool"] = cpu_baseline_pool(w, all_cores)
    else:
        line["cpu_baseline"] = None
    line["env"] = {"versions": versions(), "gpu_state": gpu_state(), "pcie": pcie_link()}
    line["input_sha256"] = input_hashes(w)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(dict(line, latency=res), f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
