"""Python binding of the lane C ABI (include/ws.h, include/ws_bench.h).

Argument marshalling only: every step of the pipeline runs in the HIP
library.  If the library is missing or cannot be loaded this module raises;
there is no fallback implementation.

Device buffers may be borrowed from any object exposing ``data_ptr()`` (a
torch tensor) or given as integer addresses.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import (POINTER, Structure, byref, c_char_p, c_double, c_float, c_int, c_int32,
                    c_size_t, c_uint8, c_void_p)

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libws.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_PKG), "include")

WS_OK = 0
WS_E_INVALID_ARG = -1
WS_E_STATE = -2
WS_E_NO_MAP_HOST = -3
WS_E_OOM = -4
WS_E_CAPTURE = -5
WS_E_HIP = -6
WS_E_NO_DEVICE = -7

RESIZE_BILINEAR = 0
RESIZE_LETTERBOX = 1
INPUT_MAPPED_HOST = 0
INPUT_DEVICE = 1
INPUT_COPY = 2
DTYPE_F32 = 0
DTYPE_F16 = 1
DTYPE_BF16 = 2
CHANNELS_RGB = 0
CHANNELS_BGR = 1
WAIT_SPIN = 0
WAIT_BLOCK = 1
CACHE_AUTO = 0
CACHE_KEEP = 1
CACHE_STREAM = 2
MAX_K = 32
STAGE_PREPROCESS = 0
STAGE_TOPK = 1
STAGE_DETECT = 2
LAUNCH_GRAPH = 0
LAUNCH_DIRECT = 1
DET_MAX_DET = 1024


class TopkEntry(Structure):
    _fields_ = [("score", c_float), ("index", c_int32)]


class Det(Structure):
    _fields_ = [("x1", c_float), ("y1", c_float), ("x2", c_float), ("y2", c_float),
                ("score", c_float), ("class_id", c_int32)]


class DetResult(Structure):
    _fields_ = [("count", c_int32), ("candidates", c_int32), ("det", Det * DET_MAX_DET)]


class LaneConfig(Structure):
    _fields_ = [
        ("device", c_int32), ("batch", c_int32),
        ("src_w", c_int32), ("src_h", c_int32),
        ("dst_w", c_int32), ("dst_h", c_int32),
        ("resize_mode", c_int32), ("input_mode", c_int32),
        ("pad_value", c_double), ("mean", c_double * 3), ("std", c_double * 3),
        ("num_scores", c_int32), ("k", c_int32),
        ("use_graph", c_int32), ("wait_mode", c_int32),
        ("input_dev", c_void_p), ("scores_dev", c_void_p), ("tensor_dev", c_void_p),
        ("rows_per_group", c_int32), ("topk_chunk", c_int32),
        ("pixels_per_thread", c_int32),
        ("tensor_dtype", c_int32), ("channel_order", c_int32), ("autotune", c_int32),
        ("det_classes", c_int32), ("det_max_det", c_int32),
        ("det_conf", c_float), ("det_iou", c_float),
        ("det_agnostic", c_int32), ("det_reserved", c_int32), ("det_head_dev", c_void_p),
        ("cache_policy", c_int32), ("reserved", c_int32),
    ]


class LaneView(Structure):
    _fields_ = [
        ("input_host", POINTER(c_uint8)), ("input_dev", c_void_p),
        ("tensor_dev", c_void_p), ("scores_dev", c_void_p),
        ("result_host", POINTER(TopkEntry)),
        ("input_bytes", c_size_t), ("tensor_bytes", c_size_t),
        ("det_head_dev", c_void_p), ("det_result_host", POINTER(DetResult)),
    ]


class LanePlan(Structure):
    _fields_ = [
        ("pre_groups", c_int32), ("pre_block", c_int32), ("rows_per_group", c_int32),
        ("pre_lds_bytes", c_int32), ("topk_groups", c_int32), ("topk_block", c_int32),
        ("topk_chunk", c_int32), ("graph_nodes", c_int32), ("pixels_per_thread", c_int32),
        ("det_anchors", c_int32), ("det_decode_groups", c_int32), ("topk_keys_per_lane", c_int32),
        ("streaming", c_int32),
    ]


class WsError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        super().__init__(f"{what}: {status_str(status)} ({status}), hip error {hip_error}")


_lib = None


def load(path: str = LIB_PATH):
    """Load libws.so (built by post_processing_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m post_processing_amd.build`")
    # PyTorch wheels carry their own HIP runtime.  Loaded after the library,
    # torch would bring a second HIP and HSA runtime into the process, and the
    # two fight over the device.  Loaded before it, the library binds to
    # torch's copy (same soname), so the process has exactly one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.ws_create_lane.argtypes = [POINTER(LaneConfig), POINTER(c_void_p), POINTER(LaneView)]
    lib.ws_create_lane.restype = c_int
    lib.ws_submit.argtypes = [c_void_p]
    lib.ws_submit.restype = c_int
    lib.ws_wait.argtypes = [c_void_p, POINTER(c_float)]
    lib.ws_wait.restype = c_int
    lib.ws_destroy.argtypes = [c_void_p]
    lib.ws_destroy.restype = c_int
    lib.ws_status_str.argtypes = [c_int]
    lib.ws_status_str.restype = c_char_p
    lib.ws_lane_hip_error.argtypes = [c_void_p]
    lib.ws_lane_hip_error.restype = c_int
    lib.ws_lane_describe.argtypes = [c_void_p, POINTER(LanePlan)]
    lib.ws_lane_describe.restype = c_int
    lib.ws_bench_replays.argtypes = [c_void_p, c_int32, POINTER(c_float), POINTER(c_float),
                                     POINTER(c_float), POINTER(c_double)]
    lib.ws_bench_replays.restype = c_int
    lib.ws_bench_lanes.argtypes = [POINTER(c_void_p), c_int32, c_int32, POINTER(c_float),
                                   POINTER(c_double)]
    lib.ws_bench_lanes.restype = c_int
    lib.ws_bench_stage.argtypes = [c_void_p, c_int32, c_int32, POINTER(c_double)]
    lib.ws_bench_stage.restype = c_int
    lib.ws_bench_stage_cold.argtypes = [c_void_p, c_int32, c_void_p, c_size_t, c_int32, c_int32,
                                        POINTER(c_float)]
    lib.ws_bench_stage_cold.restype = c_int
    lib.ws_bench_stage_rotate.argtypes = [POINTER(c_void_p), c_int32, c_int32, c_int32, c_int32,
                                          POINTER(c_double)]
    lib.ws_bench_stage_rotate.restype = c_int
    lib.ws_run_noalloc.argtypes = [POINTER(LaneConfig), c_void_p, c_void_p]
    lib.ws_run_noalloc.restype = c_int
    lib.ws_bench_launch_cost.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32,
                                         POINTER(c_float), POINTER(c_float), POINTER(c_float),
                                         POINTER(c_int32)]
    lib.ws_bench_launch_cost.restype = c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().ws_status_str(status).decode()


def declared_functions() -> list[str]:
    """Names of every function declared in include/*.h."""
    names = []
    for fn in sorted(os.listdir(INCLUDE_DIR)):
        if fn.endswith(".h"):
            with open(os.path.join(INCLUDE_DIR, fn)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \t\*]*?\b(ws_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def _addr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def make_config(*, src_w, src_h, dst_w, dst_h, batch=1, letterbox=False, pad=114.0,
                mean=(0.0, 0.0, 0.0), std=(1.0, 1.0, 1.0), num_scores=0, k=0,
                host_input=False, use_graph=True, wait_mode=WAIT_SPIN, device=0,
                input_dev=None, scores_dev=None, tensor_dev=None, rows_per_group=0,
                topk_chunk=0, pixels_per_thread=0, input_mode=None, tensor_dtype=DTYPE_F32,
                channel_order=CHANNELS_RGB, autotune=False, det_classes=0, det_max_det=300,
                det_conf=0.25, det_iou=0.45, det_agnostic=False,
                det_head_dev=None, cache_policy=CACHE_AUTO) -> LaneConfig:
    c = LaneConfig()
    c.device = device
    c.batch = batch
    c.src_w, c.src_h, c.dst_w, c.dst_h = src_w, src_h, dst_w, dst_h
    c.resize_mode = RESIZE_LETTERBOX if letterbox else RESIZE_BILINEAR
    if input_mode is None:
        input_mode = INPUT_MAPPED_HOST if host_input else INPUT_DEVICE
    c.input_mode = input_mode
    c.pad_value = float(pad)
    c.mean[:] = [float(v) for v in mean]
    c.std[:] = [float(v) for v in std]
    c.num_scores = num_scores
    c.k = k
    c.use_graph = 1 if use_graph else 0
    c.wait_mode = wait_mode
    c.input_dev = _addr(input_dev)
    c.scores_dev = _addr(scores_dev)
    c.tensor_dev = _addr(tensor_dev)
    c.rows_per_group = rows_per_group
    c.topk_chunk = topk_chunk
    c.pixels_per_thread = pixels_per_thread
    c.tensor_dtype = tensor_dtype
    c.channel_order = channel_order
    c.autotune = 1 if autotune else 0
    c.cache_policy = cache_policy
    c.det_classes = det_classes
    if det_classes:
        c.det_max_det = det_max_det
        c.det_conf = det_conf
        c.det_iou = det_iou
        c.det_agnostic = 1 if det_agnostic else 0
        c.det_head_dev = _addr(det_head_dev)
    return c


class Lane:
    """One pipeline lane (ws_create_lane ... ws_destroy)."""

    def __init__(self, cfg: LaneConfig):
        self._lib = load()
        self.cfg = cfg
        self.view = LaneView()
        h = c_void_p()
        rc = self._lib.ws_create_lane(byref(cfg), byref(h), byref(self.view))
        if rc != WS_OK:
            raise WsError(rc, "ws_create_lane")
        self.handle = h

    # -- per-frame calls --------------------------------------------------
    def submit(self) -> int:
        return self._lib.ws_submit(self.handle)

    def wait(self) -> tuple[int, float]:
        ms = c_float(0.0)
        rc = self._lib.ws_wait(self.handle, byref(ms))
        return rc, ms.value

    def run(self) -> float:
        """submit + wait; returns the GPU event time in ms (raises on error)."""
        rc = self.submit()
        if rc != WS_OK:
            raise WsError(rc, "ws_submit", self.hip_error())
        rc, ms = self.wait()
        if rc != WS_OK:
            raise WsError(rc, "ws_wait", self.hip_error())
        return ms

    # -- buffers ----------------------------------------------------------
    def input_host_array(self) -> np.ndarray:
        """The producer's host input slot (mapped or copy mode) as a writable
        uint8 [B][H][W][3] view."""
        if not self.view.input_host:
            raise RuntimeError("lane has no host input slot")
        c = self.cfg
        flat = np.ctypeslib.as_array(self.view.input_host, shape=(self.view.input_bytes,))
        return flat.reshape(c.batch, c.src_h, c.src_w, 3)

    def result(self) -> tuple[np.ndarray, np.ndarray]:
        """Copy of the result slot: (float32 scores[k], int32 indices[k])."""
        k = self.cfg.k
        if k == 0 or not self.view.result_host:
            raise RuntimeError("lane has no Top-K stage")
        raw = np.ctypeslib.as_array(ctypes.cast(self.view.result_host, POINTER(ctypes.c_uint32)),
                                    shape=(2 * k,)).copy()
        return raw[0::2].view(np.float32), raw[1::2].view(np.int32)

    def result_slot_words(self) -> np.ndarray:
        """Writable uint32 view of the mapped result slot (score bits, index)
        x K, e.g. to overwrite it with a marker before a replay."""
        if self.cfg.k == 0 or not self.view.result_host:
            raise RuntimeError("lane has no Top-K stage")
        return np.ctypeslib.as_array(ctypes.cast(self.view.result_host, POINTER(ctypes.c_uint32)),
                                     shape=(2 * self.cfg.k,))

    def detection_slot_words(self) -> np.ndarray:
        """Writable uint32 view of the whole mapped detection slot."""
        if not self.view.det_result_host:
            raise RuntimeError("lane has no detection stage")
        return np.ctypeslib.as_array(ctypes.cast(self.view.det_result_host,
                                                 POINTER(ctypes.c_uint32)),
                                     shape=(ctypes.sizeof(DetResult) // 4,))

    def detections(self) -> tuple[np.ndarray, np.ndarray, np.ndarray, int]:
        """Copy of the detection slot: (float32 boxes[n][4], float32 scores[n],
        int32 classes[n], number of candidates)."""
        if not self.view.det_result_host:
            raise RuntimeError("lane has no detection stage")
        r = self.view.det_result_host.contents
        n = r.count
        raw = np.ctypeslib.as_array(ctypes.cast(ctypes.addressof(r.det), POINTER(ctypes.c_uint32)),
                                    shape=(6 * n,)).copy().reshape(n, 6)
        return (raw[:, :4].view(np.float32).copy(), raw[:, 4].view(np.float32).copy(),
                raw[:, 5].view(np.int32).copy(), int(r.candidates))

    def plan(self) -> dict:
        p = LanePlan()
        rc = self._lib.ws_lane_describe(self.handle, byref(p))
        if rc != WS_OK:
            raise WsError(rc, "ws_lane_describe")
        return {name: getattr(p, name) for name, _ in LanePlan._fields_}

    def hip_error(self) -> int:
        return self._lib.ws_lane_hip_error(self.handle)

    def bench(self, replays: int, host: bool = False):
        """Native submit/wait loop: (gpu_ms per replay, wall seconds), plus
        the host microseconds per replay (submit to wait's return) and the
        part of it spent inside ws_submit, when `host` is set."""
        ms = (c_float * replays)()
        us = (c_float * replays)() if host else None
        sub = (c_float * replays)() if host else None
        wall = c_double(0.0)
        rc = self._lib.ws_bench_replays(self.handle, replays, ms, us, sub, byref(wall))
        if rc != WS_OK:
            raise WsError(rc, "ws_bench_replays", self.hip_error())
        out = np.ctypeslib.as_array(ms).copy(), wall.value
        if not host:
            return out
        return out + (np.ctypeslib.as_array(us).copy(), np.ctypeslib.as_array(sub).copy())

    def time_stage(self, stage: int, launches: int) -> float:
        """Mean ms per direct launch of one stage's kernel (native loop)."""
        ms = c_double(0.0)
        rc = self._lib.ws_bench_stage(self.handle, stage, launches, byref(ms))
        if rc != WS_OK:
            raise WsError(rc, "ws_bench_stage", self.hip_error())
        return ms.value

    def time_stage_cold(self, stage: int, flush, flush_bytes: int, launches: int,
                        write: bool = False) -> np.ndarray:
        """ms per launch of one stage, each launch after a flush kernel over
        `flush_bytes` of the device buffer `flush` (native loop)."""
        ms = (c_float * launches)()
        rc = self._lib.ws_bench_stage_cold(self.handle, stage, _addr(flush), flush_bytes,
                                           1 if write else 0, launches, ms)
        if rc != WS_OK:
            raise WsError(rc, "ws_bench_stage_cold", self.hip_error())
        return np.ctypeslib.as_array(ms).copy()

    def destroy(self) -> None:
        if self.handle:
            self._lib.ws_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


NOALLOC_SCRATCH_BYTES = 1 << 20


def run_noalloc(cfg: LaneConfig, result=None, stream=None) -> int:
    """ws_run_noalloc: one frame on the caller's buffers and stream, with no
    allocation.  `result` is a device-visible address (or tensor) for K
    entries; `stream` a hipStream_t handle (int) or None.  Returns the status."""
    return load().ws_run_noalloc(byref(cfg), _addr(result), stream)


def time_stage_rotate(lanes: list[Lane], stage: int, launches: int, warmup: int = 0) -> float:
    """Mean ms per launch of one stage launched back to back over the lanes
    in turn, on the first lane's stream (native loop)."""
    lib = load()
    n = len(lanes)
    handles = (c_void_p * n)(*[ln.handle for ln in lanes])
    ms = c_double(0.0)
    rc = lib.ws_bench_stage_rotate(handles, n, stage, warmup, launches, byref(ms))
    if rc != WS_OK:
        raise WsError(rc, "ws_bench_stage_rotate", lanes[0].hip_error())
    return ms.value


def launch_cost(nodes: int, form: int, replays: int, warmup: int = 300,
                device: int = 0) -> dict:
    """Launch overhead of `nodes` empty kernels in one of the LAUNCH_* forms
    (native loop): per-round arrays in microseconds, keys launch / total / gpu."""
    lib = load()
    arrs = [(c_float * replays)() for _ in range(3)]
    err = c_int32(0)
    rc = lib.ws_bench_launch_cost(device, nodes, form, warmup, replays, *arrs, byref(err))
    if rc != WS_OK:
        raise WsError(rc, "ws_bench_launch_cost", err.value)
    return {k: np.ctypeslib.as_array(a).copy() for k, a in zip(("launch", "total", "gpu"), arrs)}


def bench_lanes(lanes: list[Lane], replays: int) -> tuple[np.ndarray, float]:
    """Drive several lanes from one native thread each: (gpu_ms [L][R], wall s)."""
    lib = load()
    n = len(lanes)
    handles = (c_void_p * n)(*[ln.handle for ln in lanes])
    ms = (c_float * (n * replays))()
    wall = c_double(0.0)
    rc = lib.ws_bench_lanes(handles, n, replays, ms, byref(wall))
    if rc != WS_OK:
        raise WsError(rc, "ws_bench_lanes")
    return np.ctypeslib.as_array(ms).copy().reshape(n, replays), wall.value
