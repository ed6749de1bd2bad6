"""GPU parity of the detection stage (decode + greedy NMS) against the
oracle, through the C ABI.

Bar: the number of candidates, and every kept box's four corners, score and
class, identical bit for bit and in keep order.  The decisions (which
anchors pass the threshold, which boxes suppress which) are integers decided
by binary32 arithmetic, and both sides do that arithmetic with the same
operations in the same order, so any difference is a bug.
"""
import dataclasses

import numpy as np
import pytest

from post_processing_amd import workloads as wl
from post_processing_amd import ws

from gpu_util import (Run, assert_detections_exact, assert_tensor_close, assert_topk_exact,
                      oracle_detections, oracle_outputs)

pytestmark = pytest.mark.gpu
F32 = np.float32


def _run_detect(w, **knobs):
    r = Run(w, host_input=False, **knobs)
    try:
        r.run()
        return r.detections(), r.outputs()
    finally:
        r.close()


def test_c3_detection_full_pipeline(gpu_lib):
    """C3's letterbox lane with the detection stage: tensor, Top-K over the
    8400 x 80 class block and the kept boxes, all from one graph replay."""
    w = wl.c3d()
    ref, rtk = oracle_outputs(w)
    rdet = oracle_detections(w)
    got, (t, tk) = _run_detect(w)
    assert_tensor_close(t, ref)
    assert_topk_exact(tk, rtk)
    assert_detections_exact(got, rdet)
    assert 0 < len(got[1]) <= 300
    print(f"c3d: {got[3]} candidates, {len(got[1])} kept")


def test_suppression_width_does_not_change_results(gpu_lib):
    """C3D keeps 69 boxes, so max_det 300 and 1,024 give the same result.
    With 8,400 anchors (16,384-key sort space) the first fits the 16-wave
    suppression kernel in LDS and the second takes the 8-wave one."""
    w = wl.c3d()
    rdet = oracle_detections(w)
    got16, _ = _run_detect(w)
    w8 = dataclasses.replace(w, det={**w.det, "max_det": 1024})
    got8, _ = _run_detect(w8)
    assert_detections_exact(got16, rdet)
    assert_detections_exact(got8, oracle_detections(w8))
    for a, b in zip(got16, got8):
        np.testing.assert_array_equal(np.asarray(a), np.asarray(b))


@pytest.mark.parametrize("seed", range(40))
def test_detect_small_random(gpu_lib, seed):
    w = wl.detect_small(seed)
    got, (t, _) = _run_detect(w)
    ref, _ = oracle_outputs(w)
    assert_tensor_close(t, ref)
    assert_detections_exact(got, oracle_detections(w))


def _uniform_head_workload(seed, nw, nh, nc, conf, iou, max_det, agnostic=False, box_scale=1.5):
    return wl.uniform_head(seed, nw, nh, nc, conf, iou, max_det, agnostic, box_scale)


# Candidate counts across the suppression kernel's sort sizes (1024 .. 16384
# keys) and both box sources (staged in the LDS the sort leaves free, up to
# about 5,400 candidates here, else read by anchor from global memory).
# One class, so about (1 - conf) * 8400 anchors are candidates.
@pytest.mark.parametrize("conf,lo,hi", [(0.92, 1, 1024), (0.82, 1025, 2048), (0.64, 2049, 4096),
                                        (0.3, 4097, 8192), (0.01, 8193, 8400)])
def test_candidate_count_layouts(gpu_lib, conf, lo, hi):
    w = _uniform_head_workload(1, 640, 640, 1, conf, 0.5, 40)
    got, _ = _run_detect(w)
    ref = oracle_detections(w)
    assert lo <= ref[3] <= hi
    assert_detections_exact(got, ref)


@pytest.mark.parametrize("agnostic", [False, True])
def test_many_kept_boxes(gpu_lib, agnostic):
    """Hundreds of kept boxes, so the suppression runs hundreds of rounds and
    the output slot fills far past the first few entries."""
    w = _uniform_head_workload(2, 1024, 512, 80, 0.75, 0.3, 1024, agnostic=agnostic,
                               box_scale=0.3)
    got, _ = _run_detect(w)
    ref = oracle_detections(w)
    assert len(ref[1]) > 100
    assert_detections_exact(got, ref)


@pytest.mark.parametrize("iou", [0.0, 1.0])
def test_iou_threshold_extremes(gpu_lib, iou):
    # 0: any overlap suppresses; 1: nothing does (IoU never exceeds 1)
    w = _uniform_head_workload(3, 256, 256, 4, 0.7, iou, 300)
    got, _ = _run_detect(w)
    ref = oracle_detections(w)
    assert_detections_exact(got, ref)
    if iou == 1.0:
        assert len(ref[1]) == min(300, ref[3])


def test_max_det_one_and_no_candidates(gpu_lib):
    w = _uniform_head_workload(4, 320, 192, 5, 0.5, 0.45, 1)
    got, _ = _run_detect(w)
    assert_detections_exact(got, oracle_detections(w))
    assert len(got[1]) == 1
    w0 = dataclasses.replace(w, head=w.head.copy())
    w0.head[64:] = 0.1
    got0, _ = _run_detect(w0, det_conf=0.5)
    assert got0[3] == 0 and len(got0[1]) == 0


def test_tied_probabilities_and_nan(gpu_lib):
    """Equal probabilities rank by anchor (the lower first); NaN never wins a
    class and an all-NaN anchor is never a candidate."""
    w = _uniform_head_workload(5, 320, 320, 6, 0.3, 0.5, 300)
    head = w.head.copy()
    rng = np.random.default_rng(7)
    A = head.shape[1]
    tie = rng.choice(A, size=A // 3, replace=False)
    head[64 + 2, tie] = F32(0.875)
    nan_cells = rng.choice(A, size=A // 5, replace=False)
    head[64 + rng.integers(0, 6, nan_cells.size), nan_cells] = np.nan
    all_nan = rng.choice(A, size=20, replace=False)
    head[64:, all_nan] = np.nan
    w = dataclasses.replace(w, head=head)
    got, _ = _run_detect(w)
    assert_detections_exact(got, oracle_detections(w))


def test_lane_owned_head_starts_empty(gpu_lib):
    """Without a borrowed head the lane owns a zero-filled one: no class
    probability exceeds a non-negative threshold, so nothing is detected."""
    import torch
    dev = torch.device("cuda:0")
    frames = torch.zeros((1, 64, 64, 3), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    cfg = ws.make_config(src_w=64, src_h=64, dst_w=64, dst_h=64, input_dev=frames,
                         det_classes=3, det_conf=0.0)
    with ws.Lane(cfg) as lane:
        assert lane.view.det_head_dev
        lane.run()
        b, s, c, n = lane.detections()
        assert n == 0 and len(s) == 0
        assert lane.plan()["det_anchors"] == 64 + 16 + 4


def test_detection_replays_are_stable(gpu_lib):
    """The candidate counter is reset inside the graph, so every replay sees
    the same candidates and keeps the same boxes."""
    w = wl.c3d()
    r = Run(w, host_input=False)
    try:
        r.run()
        first = r.detections()
        r.lane.bench(300)
        again = r.detections()
        assert_detections_exact(again, first)
        assert_detections_exact(first, oracle_detections(w))
    finally:
        r.close()


def test_detection_graph_and_direct_agree(gpu_lib):
    w = wl.detect_small(11)
    a = Run(w, host_input=False, use_graph=True)
    b = Run(w, host_input=False, use_graph=False)
    try:
        a.run()
        b.run()
        assert_detections_exact(a.detections(), b.detections())
    finally:
        a.close()
        b.close()


def test_head_rewritten_between_frames(gpu_lib):
    """A borrowed head is read afresh by every replay."""
    import torch
    w1 = wl.detect_small(2)
    r = Run(w1, host_input=False)
    try:
        r.run()
        assert_detections_exact(r.detections(), oracle_detections(w1))
        rng = np.random.default_rng(99)
        h2 = w1.head.copy()
        h2[64:] = rng.uniform(0, 1, h2[64:].shape).astype(F32)
        r.head.copy_(torch.from_numpy(h2))
        torch.cuda.synchronize()
        r.run()
        assert_detections_exact(r.detections(), oracle_detections(w1, head=h2))
    finally:
        r.close()


def test_invalid_detection_configs_rejected(gpu_lib):
    for bad in (dict(det_classes=80, dst_w=650), dict(det_classes=80, det_max_det=0),
                dict(det_classes=80, det_conf=1.0), dict(det_classes=-1)):
        cfg = ws.make_config(src_w=640, src_h=640, dst_w=bad.pop("dst_w", 640), dst_h=640,
                             **bad)
        with pytest.raises(ws.WsError):
            ws.Lane(cfg)


@pytest.mark.parametrize("variant", ["f16_tensor", "bgr_mapped_input", "copy_input_bf16"])
def test_detection_with_other_lane_options(gpu_lib, variant):
    """The detection stage reads only the head, so the other lane options
    (tensor type, producer byte order, input mode) leave its result unchanged
    bit for bit; the tensor still meets its own bar."""
    from gpu_util import assert_rounded_close
    w = wl.detect_small(7)
    ref, _ = oracle_outputs(w)
    if variant == "f16_tensor":
        r = Run(w, host_input=False, tensor_dtype=ws.DTYPE_F16)
    elif variant == "bgr_mapped_input":
        w = dataclasses.replace(w, frames=np.ascontiguousarray(w.frames[..., ::-1]))
        r = Run(w, input_mode=ws.INPUT_MAPPED_HOST, channel_order=ws.CHANNELS_BGR)
    else:
        r = Run(w, input_mode=ws.INPUT_COPY, tensor_dtype=ws.DTYPE_BF16)
    try:
        r.run()
        assert_detections_exact(r.detections(), oracle_detections(w))
        t, _ = r.outputs()
        if variant == "bgr_mapped_input":
            assert_tensor_close(t, ref)
        else:
            assert_rounded_close(t, ref, "f16" if variant == "f16_tensor" else "bf16")
    finally:
        r.close()


def test_detection_at_the_class_limit(gpu_lib):
    """4096 classes: each decode wave scans 1024 of them."""
    rng = np.random.default_rng(4096)
    nc, nw, nh = 4096, 64, 64
    A = wl.head_anchor_grid(nw, nh)[0].size
    head = np.empty((64 + nc, A), F32)
    head[:64] = rng.normal(0.0, 1.5, (64, A))
    head[64:] = rng.uniform(0.0, 0.9, (nc, A))
    winners = rng.integers(0, nc, A)
    head[64 + winners, np.arange(A)] = rng.uniform(0.9, 1.0, A).astype(F32)
    frames = rng.integers(0, 256, size=(1, nh, nw, 3), dtype=np.uint8)
    w = wl.Workload("classes4096", nw, nh, nw, nh, wl.RESIZE, (0.0, 0.0, 0.0), (1.0, 1.0, 1.0),
                    114.0, 0, frames, None, head=head,
                    det=dict(nc=nc, conf=0.95, iou=0.5, max_det=300, agnostic=False))
    got, _ = _run_detect(w)
    ref = oracle_detections(w)
    assert ref[3] > 10
    assert_detections_exact(got, ref)


def test_detection_near_the_anchor_limit(gpu_lib):
    """A 1024 x 768 network input: 16,128 anchors (the limit is 16,384)."""
    nw, nh = 1024, 768
    region = (0, 0, nw, nh)
    head, planted = wl.detection_head(np.random.default_rng(16128), nw, nh, 3, region, 10)
    frames = np.random.default_rng(1).integers(0, 256, size=(1, nh, nw, 3), dtype=np.uint8)
    w = wl.Workload("anchors16128", nw, nh, nw, nh, wl.RESIZE, (0.0, 0.0, 0.0), (1.0, 1.0, 1.0),
                    114.0, 0, frames, None, head=head,
                    det=dict(nc=3, conf=0.25, iou=0.45, max_det=300, agnostic=False))
    assert head.shape[1] == 16128
    got, _ = _run_detect(w)
    assert_detections_exact(got, oracle_detections(w))


@pytest.mark.parametrize("case", ["c3d"] + [f"small{i}" for i in range(40)])
def test_detection_matches_float64_definitions(gpu_lib, case):
    """The GPU's kept boxes against greedy suppression on the float64
    definitions directly (not through the oracle's binary32 path): the same
    candidate count and rank order, each box within the derived binary32
    bound of its softmax-expectation box mapped to source pixels, and every
    keep/suppress decision equal to the exact-rational IoU decision wherever
    |IoU - threshold| exceeds the binary32 error bound.  Decisions inside
    that band are counted and printed."""
    from detect_exact import check_against_definitions
    from gpu_util import workload_region
    w = wl.c3d() if case == "c3d" else wl.detect_small(int(case[5:]))
    d = w.det
    got, _ = _run_detect(w)
    in_band = check_against_definitions(got, w.head, w.src_w, w.src_h, w.dst_w, w.dst_h,
                                        workload_region(w), d["conf"], d["iou"], d["max_det"],
                                        d["agnostic"])
    print(f"{case}: {got[3]} candidates, {len(got[1])} kept, {in_band} decisions in the band")
