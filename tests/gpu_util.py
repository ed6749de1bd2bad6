"""Helpers shared by the GPU parity tests: run a workload through the C ABI and
compute the oracle's answer for it."""
import numpy as np

from oracle import letterbox_region, preprocess_batch, topk
from oracle import detect as odet
from post_processing_amd import workloads as wl
from post_processing_amd import ws

TOL = 1e-5   # absolute bound on |tensor - oracle| for the FP32 tensor


def oracle_outputs(w: wl.Workload):
    ref = preprocess_batch(w.frames, w.dst_w, w.dst_h, w.mean, w.std,
                           letterbox=(w.mode == wl.LETTERBOX), pad=w.pad)
    tk = topk(w.scores, w.k) if w.k else None
    return ref, tk


def workload_region(w: wl.Workload):
    """(left, top, width, height) of the image inside the network input."""
    if w.mode == wl.LETTERBOX:
        return letterbox_region(w.src_w, w.src_h, w.dst_w, w.dst_h)
    return (0, 0, w.dst_w, w.dst_h)


def oracle_detections(w: wl.Workload, head=None, **override):
    """The oracle's decode + NMS for a workload's head (or `head`), with
    optional threshold overrides."""
    d = dict(w.det)
    d.update(override)
    return odet.detect(w.head if head is None else head, w.src_w, w.src_h, w.dst_w, w.dst_h,
                       workload_region(w), d["nc"], d["conf"], d["iou"], d["max_det"],
                       d["agnostic"])


class Run:
    """A lane built for a workload, with borrowed torch buffers kept alive."""

    def __init__(self, w: wl.Workload, host_input=None, use_graph=True, input_mode=None,
                 tensor_dtype=ws.DTYPE_F32, **knobs):
        import torch
        self.w = w
        self.host_input = w.host_input if host_input is None else host_input
        if input_mode is None:
            input_mode = ws.INPUT_MAPPED_HOST if self.host_input else ws.INPUT_DEVICE
        self.host_input = input_mode != ws.INPUT_DEVICE
        dev = torch.device("cuda:0")
        tdt = {ws.DTYPE_F32: torch.float32, ws.DTYPE_F16: torch.float16,
               ws.DTYPE_BF16: torch.bfloat16}[tensor_dtype]
        self.tensor = torch.empty((w.batch, 3, w.dst_h, w.dst_w), dtype=tdt, device=dev)
        self.tensor.fill_(float("nan"))
        self.scores = None
        if w.k:
            self.scores = torch.from_numpy(w.scores).to(dev)
        self.head = None
        det = {}
        if w.head is not None:
            self.head = torch.from_numpy(np.ascontiguousarray(w.head)).to(dev)
            det = dict(det_classes=w.det["nc"], det_max_det=w.det["max_det"],
                       det_conf=w.det["conf"], det_iou=w.det["iou"],
                       det_agnostic=w.det["agnostic"], det_head_dev=self.head)
            det.update({k: knobs.pop(k) for k in list(knobs) if k.startswith("det_")})
        self.frames = None
        if not self.host_input:
            self.frames = torch.from_numpy(np.ascontiguousarray(w.frames)).to(dev)
        torch.cuda.synchronize()
        cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h,
                             batch=w.batch, letterbox=(w.mode == wl.LETTERBOX), pad=w.pad,
                             mean=w.mean, std=w.std, num_scores=w.num_scores, k=w.k,
                             input_mode=input_mode, use_graph=use_graph, tensor_dtype=tensor_dtype,
                             input_dev=self.frames, scores_dev=self.scores,
                             tensor_dev=self.tensor, **det, **knobs)
        self.lane = ws.Lane(cfg)
        if self.host_input:
            self.lane.input_host_array()[...] = w.frames

    def run(self):
        ms = self.lane.run()
        return ms

    def outputs(self):
        t = self.tensor.float().cpu().numpy()
        tk = self.lane.result() if self.w.k else None
        return t, tk

    def detections(self):
        return self.lane.detections()

    def close(self):
        self.lane.destroy()


def assert_tensor_close(got, ref, tol=TOL):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite values in the tensor"
    err = np.abs(got.astype(np.float64) - ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"max |err| {err.max():.3e} at {worst}"
    return float(err.max())


MANTISSA_BITS = {"f16": 10, "bf16": 7}


def assert_rounded_close(got, ref, fmt, slack=2e-6):
    """A 16-bit tensor: every element within half an ulp of the output format
    (at the exact value) plus the FP32 arithmetic's slack of the exact value,
    i.e. the correctly rounded value or, at a near-tie, its neighbour."""
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite values in the tensor"
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - MANTISSA_BITS[fmt])
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > 0.5 * ulp + slack
    assert not bad.any(), f"{int(bad.sum())} elements off; worst {err[bad].max():.3e}"
    return float((err / ulp).max())


def assert_topk_exact(got, ref):
    gv, gi = got
    rv, ri = ref
    np.testing.assert_array_equal(gi, ri)
    np.testing.assert_array_equal(gv.view(np.uint32), rv.view(np.uint32))


def assert_detections_exact(got, ref):
    """Kept boxes, scores and classes identical bit for bit, in keep order,
    and the same number of candidates."""
    gb, gs, gc, gn = got
    rb, rs, rc, rn = ref
    assert gn == rn, f"candidates: gpu {gn}, oracle {rn}"
    assert len(gs) == len(rs), f"kept: gpu {len(gs)}, oracle {len(rs)}"
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(gb.view(np.uint32), rb.astype(np.float32).view(np.uint32))
