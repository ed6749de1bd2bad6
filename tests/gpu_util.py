"""Helpers shared by the GPU parity tests: run a workload through the C ABI and
compute the oracle's answer for it."""
import numpy as np

from oracle import preprocess_batch, topk
from post_processing_amd import workloads as wl
from post_processing_amd import ws

TOL = 1e-5   # absolute bound on |tensor - oracle| for the FP32 tensor


def oracle_outputs(w: wl.Workload):
    ref = preprocess_batch(w.frames, w.dst_w, w.dst_h, w.mean, w.std,
                           letterbox=(w.mode == wl.LETTERBOX), pad=w.pad)
    tk = topk(w.scores, w.k) if w.k else None
    return ref, tk


class Run:
    """A lane built for a workload, with borrowed torch buffers kept alive."""

    def __init__(self, w: wl.Workload, host_input=None, use_graph=True, input_mode=None, **knobs):
        import torch
        self.w = w
        self.host_input = w.host_input if host_input is None else host_input
        if input_mode is None:
            input_mode = ws.INPUT_MAPPED_HOST if self.host_input else ws.INPUT_DEVICE
        self.host_input = input_mode != ws.INPUT_DEVICE
        dev = torch.device("cuda:0")
        self.tensor = torch.empty((w.batch, 3, w.dst_h, w.dst_w), dtype=torch.float32, device=dev)
        self.tensor.fill_(float("nan"))
        self.scores = None
        if w.k:
            self.scores = torch.from_numpy(w.scores).to(dev)
        self.frames = None
        if not self.host_input:
            self.frames = torch.from_numpy(np.ascontiguousarray(w.frames)).to(dev)
        torch.cuda.synchronize()
        cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h,
                             batch=w.batch, letterbox=(w.mode == wl.LETTERBOX), pad=w.pad,
                             mean=w.mean, std=w.std, num_scores=w.num_scores, k=w.k,
                             input_mode=input_mode, use_graph=use_graph,
                             input_dev=self.frames, scores_dev=self.scores,
                             tensor_dev=self.tensor, **knobs)
        self.lane = ws.Lane(cfg)
        if self.host_input:
            self.lane.input_host_array()[...] = w.frames

    def run(self):
        ms = self.lane.run()
        return ms

    def outputs(self):
        t = self.tensor.cpu().numpy()
        tk = self.lane.result() if self.w.k else None
        return t, tk

    def close(self):
        self.lane.destroy()


def assert_tensor_close(got, ref, tol=TOL):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite values in the tensor"
    err = np.abs(got.astype(np.float64) - ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"max |err| {err.max():.3e} at {worst}"
    return float(err.max())


def assert_topk_exact(got, ref):
    gv, gi = got
    rv, ri = ref
    np.testing.assert_array_equal(gi, ri)
    np.testing.assert_array_equal(gv.view(np.uint32), rv.view(np.uint32))
