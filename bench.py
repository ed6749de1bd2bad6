"""Benchmark of the fixed-shape frame pipeline on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one replay of a lane's graph (fused preprocess, then exact Top-K)
between the lane's two GPU events, driven by the native submit/wait loop; the
inputs are resident (device memory, or the mapped host slot for the
host-input lanes) before the timed region starts.  Prints ONE JSON line.

Workloads (synthetic, seeded; shapes of the pages' classifier and detector
inputs):
  c2   1920x1080 RGB8 -> 224x224 ImageNet-normalised + Top-5 of 1000 (default)
  c1   64x48 -> 32x32 + Top-5 of 1000 with planted ties
  c3   1280x720 -> 640x640 letterbox (pad 114, /255) + Top-32 of 8400x80
  c4   3840x2160 -> 384x384 + Top-32 of 21843 with 1% duplicates
  c5l  8 lanes, one host thread each, 1920x1080 from mapped host memory, Top-10
  c5t  64 frames 1280x720 -> 224x224 in one launch (preprocess only)
  c3d  c3's lane plus in-graph detection decode + NMS over a synthetic
       8400-anchor, 80-class head (conf 0.25, IoU 0.45, at most 300 boxes)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# (two passes), scaled by what the same counters read for a plain 256 MiB copy
# (x2.0 read, x1.0 write).  Valid only for the kernel sources they were taken
# on: reported as null once those sources change.
MEASURED_TRAFFIC = {
    "kernel_sha256_prefix": "6e458a1100d57905",
    # c5t: FETCH 53,787.5 KiB x 2.0 + WRITE 37,632.0 KiB per launch (67 launches, median)
    "c5t_64x1280x720_to_224": {"preprocess": 110_156_800 + 38_535_168},
    # c2: preprocess FETCH 1,287.5 KiB x 2.0 + WRITE 588.0 KiB; Top-K 13.6875 KiB x 2.0 +
    # 0.0625 KiB (272 launches each, median)
    "c2_1920x1080_to_224": {"preprocess": 2_636_800 + 602_112, "topk": 28_032 + 64},
}


def kernel_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    # The sources the preprocess and Top-K kernels compile from (the
    # detection kernels' file is not among them).
    for name in ("ws_kernels.hip", "ws_kernels.h", "ws_lanes.h"):
        with open(os.path.join(ROOT, "post_processing_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    if kernel_sources_sha()[:16] != MEASURED_TRAFFIC["kernel_sha256_prefix"]:
        return None
    return MEASURED_TRAFFIC.get(workload, {}).get(kernel)


# ---------------------------------------------------------------------------
# Algorithmic bytes (what the method must move at minimum, per frame).

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
    64 box logits, and writes a 16-byte box and an 8-byte key per candidate;
    suppression reads those back and writes 24 bytes per kept box."""
    nc, a = w.det["nc"], w.head.shape[1]
    return 4 * nc * a + candidates * (256 + 24 + 24) + 24 * kept + 8


# ---------------------------------------------------------------------------

def pct(a, q):
    return float(np.percentile(a, q))


def lat_stats(ms: np.ndarray) -> dict:
    us = ms.astype(np.float64) * 1e3
    return {"p50_us": pct(us, 50), "p99_us": pct(us, 99), "mean_us": float(us.mean()),
            "max_us": float(us.max()), "min_us": float(us.min()),
            "p99_over_p50": pct(us, 99) / pct(us, 50)}


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


def stage_roofline(lane, w, launches: int) -> dict:
    """Per-kernel mean duration from back-to-back launches between HIP events
    on the lane's stream, and the algorithmic bandwidth it implies."""
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


def roofline_obj(stages: dict, workload: str) -> dict:
    """The preprocess kernel against HBM: it is the stage that moves the
    frame and the tensor, and the one the metric names.  Top-K (a few KB to
    2.7 MB) and detection are latency-bound single- or few-workgroup chains,
    which a bandwidth roofline does not describe; their times are in
    `kernels`, and `slowest_stage` names the stage that took longest."""
    name = "preprocess"
    st = stages[name]
    slow = max(stages, key=lambda s: stages[s]["us"])
    return {"kernel": name, "bound": "hbm", "achieved": round(st["gbs"], 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(st["gbs"] / HBM_PEAK_GBS, 5),
            "traffic": measured_traffic(workload, name), "bytes_per_launch": st["bytes"],
            "us_per_launch": round(st["us"], 3),
            "slowest_stage": {"kernel": slow, "us_per_launch": round(stages[slow]["us"], 3)}}


def run_single(w, torch, steps, warmup, use_graph=True):
    lane = make_lane(w, torch, use_graph=use_graph)
    lane.bench(warmup)
    torch.cuda.synchronize()
    ms, wall, host_us = lane.bench(steps, host=True)
    torch.cuda.synchronize()
    res = {"frames_per_s": steps * w.batch / wall, "wall_s": wall, **lat_stats(ms),
           "host_p50_us": pct(host_us, 50), "host_p99_us": pct(host_us, 99),
           "plan": lane.plan()}
    return lane, res


def cold_launches(lane, torch, n: int, flush_bytes: int = 1 << 30) -> np.ndarray:
    """Single preprocess launches (HIP events around one direct launch), each
    after reading a >= 1 GiB buffer, so no cache level holds the frame or the
    tensor.  The evicting pass only reads (the buffer is written once, before
    the loop), so no dirty lines are left behind for the timed launch to write
    back.  Returns microseconds per launch (dispatch overhead included)."""
    from post_processing_amd import ws
    flush = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    out = []
    for _ in range(n):
        flush.sum()
        torch.cuda.synchronize()
        out.append(lane.time_stage(ws.STAGE_PREPROCESS, 1) * 1e3)
    del flush
    return np.asarray(out, dtype=np.float64)


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


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    from threadpoolctl import threadpool_limits

    from oracle import letterbox_region, preprocess_batch, topk
    from oracle import detect as odet
    with threadpool_limits(1):
        def one():
            preprocess_batch(w.frames, w.dst_w, w.dst_h, w.mean, w.std,
                             letterbox=(w.mode == 1), pad=w.pad)
            if w.k:
                topk(w.scores, w.k)
            if w.head is not None:
                reg = (letterbox_region(w.src_w, w.src_h, w.dst_w, w.dst_h) if w.mode == 1
                       else (0, 0, w.dst_w, w.dst_h))
                odet.detect(w.head, w.src_w, w.src_h, w.dst_w, w.dst_h, reg, w.det["nc"],
                            w.det["conf"], w.det["iou"], w.det["max_det"], w.det["agnostic"])
        one()   # warm-up
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            one()
            times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": round(w.batch / med, 3), "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": (f"{len(times)} calls of {w.batch} frame{'s' if w.batch > 1 else ''} of "
                       f"{w.name} (float64 preprocess"
                       f"{' + stable-sort Top-K' if w.k else ''}"
                       f"{' + binary32 decode/NMS' if w.head is not None else ''}), median "
                       f"{med * 1e3:.1f} ms per call after 1 warm-up, 1 thread"),
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

def versions() -> dict:
    out = {"python": platform.python_version(), "numpy": np.__version__}
    try:
        import torch
        out["torch"] = torch.__version__
        out["hip"] = getattr(torch.version, "hip", None)
    except Exception:
        pass
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True,
                           timeout=30)
        out["hipcc"] = r.stdout.splitlines()[0] if r.stdout else None
    except Exception:
        pass
    # The HIP runtime the lanes actually run on (the first one loaded wins).
    try:
        with open("/proc/self/maps") as f:
            out["hip_runtime_files"] = sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        pass
    return out


def gpu_state() -> dict:
    for cmd in (["amd-smi", "metric", "--json"], ["rocm-smi", "--showclocks", "--showtemp",
                                                    "--showpower", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            if r.returncode == 0 and r.stdout.strip():
                return {"tool": cmd[0], "raw": r.stdout[:4000]}
        except Exception:
            continue
    return {}


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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="c2",
                    choices=["c1", "c2", "c3", "c4", "c5l", "c5t", "c3d", "copy"])
    ap.add_argument("--copy-mib", type=int, default=256,
                    help="copy workload: bytes per device-to-device copy (MiB)")
    ap.add_argument("--stage-launches", type=int, default=500)
    ap.add_argument("--rows-per-group", type=int, default=0, help="preprocess tuning knob (0 = auto)")
    ap.add_argument("--topk-chunk", type=int, default=0, help="Top-K tuning knob (0 = auto)")
    ap.add_argument("--dtype", default="f32", choices=["f32", "f16", "bf16"],
                    help="tensor element type (arithmetic stays FP32)")
    ap.add_argument("--input", default=None, choices=["device", "mapped", "copy"],
                    help="override the workload's input mode")
    ap.add_argument("--pixels-per-thread", type=int, default=0,
                    help="preprocess tuning knob: 1, 2 or 4 (0 = auto)")
    ap.add_argument("--autotune", action="store_true",
                    help="let each lane time candidate launch geometries at create")
    ap.add_argument("--lanes", type=int, default=1,
                    help="lanes driven at once, one host thread each, each with its own "
                         "buffers (not c5l, which is eight lanes): one lane's work runs while "
                         "another's is launched")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-direct", action="store_true", help="skip the direct-launch comparison")
    ap.add_argument("--report", default=None, help="also write a detailed JSON report here")
    ap.add_argument("--graph-packet-capture", choices=["off", "runtime-default"],
                    default="runtime-default",
                    help="HIP runtime graph mode (DEBUG_CLR_GRAPH_PACKET_CAPTURE), read once when "
                         "HIP starts; 'off' only for comparison")
    ap.add_argument("--pin-core", type=int, default=-2,
                    help="run the submit/wait loop on this host core (-2: the last core this "
                         "process may use; -1: no pinning); single-lane workloads only")
    args = ap.parse_args(argv)
    if args.graph_packet_capture == "off":
        # Must be in the environment before torch (or anything else) starts HIP.
        os.environ["DEBUG_CLR_GRAPH_PACKET_CAPTURE"] = "0"
    pinned = None
    all_cores = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
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
    from post_processing_amd import workloads as wl
    from post_processing_amd import ws
    ws.load()

    KNOBS.update(rows_per_group=args.rows_per_group, topk_chunk=args.topk_chunk,
                 pixels_per_thread=args.pixels_per_thread, autotune=args.autotune)
    TENSOR["dtype"] = args.dtype
    if args.input:
        INPUT_OVERRIDE["mode"] = {"device": ws.INPUT_DEVICE, "mapped": ws.INPUT_MAPPED_HOST,
                                  "copy": ws.INPUT_COPY}[args.input]
    name = args.workload
    if name == "copy":
        return copy_calibration(torch, args)
    t_gen = time.perf_counter()
    if name == "c5l":
        work = [wl.c5_lane(i) for i in range(8)]
        w = work[0]
    elif name == "c5t":
        w = wl.c5_throughput(64)
    elif name == "c3d":
        w = wl.c3d()
    else:
        w = wl.ALL_CONFIGS[name]()
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] inputs for {name} ready in {gen_s:.1f} s", file=sys.stderr, flush=True)

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
    if multi:
        lanes = [make_lane(x, torch) for x in (work if name == "c5l" else [w] * args.lanes)]
        ws.bench_lanes(lanes, args.warmup)
        torch.cuda.synchronize()
        ms, wall = ws.bench_lanes(lanes, args.steps)
        torch.cuda.synchronize()
        frames = len(lanes) * w.batch * args.steps
        res = {"frames_per_s": frames / wall, "wall_s": wall, **lat_stats(ms.ravel()),
               "per_lane_p50_us": [pct(m * 1e3, 50) for m in ms],
               "plan": lanes[0].plan()}
        stages = stage_roofline(lanes[0], w, args.stage_launches)
        pb = preprocess_bytes(w)
        if name == "c5l":
            extra["mapped_host_read_gbs"] = pb["read"] / (stages["preprocess"]["us"] * 1e-6) / 1e9
            extra["pinned_h2d_copy_gbs"] = pinned_h2d_gbs(torch)
        lane = lanes[0]
        steps_total = len(lanes) * args.steps
    else:
        lane, res = run_single(w, torch, args.steps, args.warmup)
        stages = stage_roofline(lane, w, args.stage_launches)
        steps_total = args.steps
        if name == "c5t":
            cold = cold_launches(lane, torch, 20)
            pb = preprocess_bytes(w)
            extra["cold_preprocess_us_p50"] = float(np.median(cold))
            extra["cold_hbm_gbs"] = pb["total"] / (np.median(cold) * 1e-6) / 1e9
            extra["cold_frac_of_hbm_peak"] = extra["cold_hbm_gbs"] / HBM_PEAK_GBS
        if lane.cfg.input_mode != ws.INPUT_DEVICE:
            pb = preprocess_bytes(w)
            if lane.cfg.input_mode == ws.INPUT_MAPPED_HOST:
                extra["mapped_host_read_gbs"] = (pb["read"] / (stages["preprocess"]["us"] * 1e-6)
                                                 / 1e9)
            extra["pinned_h2d_copy_gbs"] = pinned_h2d_gbs(torch)
        if not args.no_direct and name != "c5t":
            dl, dres = run_single(w, torch, min(args.steps, 2000), min(args.warmup, 200),
                                  use_graph=False)
            extra["direct_launch"] = {k: dres[k] for k in ("frames_per_s", "p50_us", "p99_us")}
            dl.destroy()

    roof = roofline_obj(stages, w.name)
    pb = preprocess_bytes(w)
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
        "config": {"workload": w.name if name != "c5l" else "c5l_8lanes_1920x1080_to_224_mapped",
                   "frames_per_step": w.batch, "src": [w.src_w, w.src_h],
                   "dst": [w.dst_w, w.dst_h], "letterbox": w.mode == 1,
                   "topk": {"n": w.num_scores, "k": w.k} if w.k else None,
                   "detect": ({"anchors": int(w.head.shape[1]), **{k: w.det[k] for k in
                              ("nc", "conf", "iou", "max_det")}} if w.head is not None else None),
                   "input": args.input or ("mapped" if (w.host_input or name == "c5l") else "device"),
                   "graph": True, "lanes": 8 if name == "c5l" else args.lanes,
                   "graph_packet_capture": args.graph_packet_capture,
                   "host_core": pinned,
                   "parallelism": "single_gpu"},
        "p50_us": round(res["p50_us"], 3),
        "p99_us": round(res["p99_us"], 3),
        "p99_over_p50": round(res["p99_over_p50"], 4),
        # Host view of the same replays: just before ws_submit to ws_wait's return.
        "host_submit_to_return_us": ({"p50": round(res["host_p50_us"], 3),
                                      "p99": round(res["host_p99_us"], 3)}
                                     if "host_p50_us" in res else None),
        "preprocess_gbs": round(stages["preprocess"]["gbs"], 2),
        "preprocess_frac_of_hbm_peak": round(stages["preprocess"]["gbs"] / HBM_PEAK_GBS, 5),
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
    if args.report:
        rep = dict(line)
        rep["latency"] = {k: res[k] for k in res if k.endswith("_us") or k.startswith("p99")}
        rep["versions"] = versions()
        rep["gpu_state"] = gpu_state()
        rep["input_sha256"] = {"frames": wl.sha256(w.frames),
                               "scores": wl.sha256(w.scores) if w.k else None}
        with open(args.report, "w") as f:
            json.dump(rep, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
