"""The allocation-free entry point (ws_run_noalloc) against the lane path
(ws_submit) on the same inputs, through the C ABI: tensors bit for bit and
Top-K indices and value bits identical, and both against the oracle.  Two
calls in a row, the second with a smaller input, so the second reuses the
scratch array the first left filled."""
import numpy as np
import pytest

from oracle import topk
from post_processing_amd import workloads as wl
from post_processing_amd import ws

from gpu_util import Run, assert_tensor_close, assert_topk_exact, oracle_outputs

pytestmark = pytest.mark.gpu


def _noalloc(w):
    """Run `w` through ws_run_noalloc on fresh torch buffers on torch's
    current stream; returns (tensor, (values, indices))."""
    import torch
    dev = torch.device("cuda:0")
    frames = torch.from_numpy(np.ascontiguousarray(w.frames)).to(dev)
    scores = torch.from_numpy(w.scores).to(dev)
    tensor = torch.full((w.batch, 3, w.dst_h, w.dst_w), float("nan"), dtype=torch.float32,
                        device=dev)
    result = torch.full((2 * w.k,), -1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h,
                         batch=w.batch, letterbox=(w.mode == wl.LETTERBOX), pad=w.pad,
                         mean=w.mean, std=w.std, num_scores=w.num_scores, k=w.k,
                         input_mode=ws.INPUT_DEVICE, input_dev=frames, scores_dev=scores,
                         tensor_dev=tensor)
    stream = torch.cuda.current_stream().cuda_stream
    rc = ws.run_noalloc(cfg, result, stream)
    assert rc == ws.WS_OK, ws.status_str(rc)
    torch.cuda.synchronize()
    raw = result.cpu().numpy()
    return tensor.cpu().numpy(), (raw[0::2].view(np.float32), raw[1::2].view(np.int32))


@pytest.mark.parametrize("first,second", [("c3", "c4")])
def test_noalloc_matches_lane_on_two_calls(gpu_lib, first, second):
    for name in (first, second):            # the second input is the smaller one
        w = wl.ALL_CONFIGS[name]()
        ref, rtk = oracle_outputs(w)
        r = Run(w, host_input=False)
        try:
            groups = r.lane.plan()["topk_groups"]
            assert groups > 1                 # the partial lists go through the scratch array
            r.run()
            lt, ltk = r.outputs()
        finally:
            r.close()
        nt, ntk = _noalloc(w)
        np.testing.assert_array_equal(nt.view(np.uint32), lt.view(np.uint32))
        assert_topk_exact(ntk, ltk)
        assert_tensor_close(nt, ref)
        assert_topk_exact(ntk, rtk)


def test_noalloc_rejects_plans_beyond_the_scratch_and_missing_buffers(gpu_lib):
    import torch
    dev = torch.device("cuda:0")
    n = 40_000_000                           # 4,883 lists of 32 keys: more than 1 MiB
    scores = torch.zeros(n, dtype=torch.float32, device=dev)
    frames = torch.zeros((1, 4, 4, 3), dtype=torch.uint8, device=dev)
    tensor = torch.zeros((1, 3, 4, 4), dtype=torch.float32, device=dev)
    result = torch.zeros(64, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    base = dict(src_w=4, src_h=4, dst_w=4, dst_h=4, input_mode=ws.INPUT_DEVICE)
    cfg = ws.make_config(**base, num_scores=n, k=32, input_dev=frames, scores_dev=scores,
                         tensor_dev=tensor)
    assert ws.run_noalloc(cfg, result, None) == ws.WS_E_INVALID_ARG
    cfg = ws.make_config(**base, num_scores=1000, k=5, input_dev=frames, scores_dev=scores,
                         tensor_dev=tensor)
    assert ws.run_noalloc(cfg, None, None) == ws.WS_E_INVALID_ARG          # no result buffer
    cfg = ws.make_config(**base, input_dev=frames, tensor_dev=None)
    assert ws.run_noalloc(cfg, None, None) == ws.WS_E_INVALID_ARG          # no tensor
    cfg = ws.make_config(src_w=4, src_h=4, dst_w=4, dst_h=4, host_input=True, tensor_dev=tensor)
    assert ws.run_noalloc(cfg, None, None) == ws.WS_E_INVALID_ARG          # mapped input
    # Within the limit the same call runs (one workgroup: no scratch needed).
    cfg = ws.make_config(**base, num_scores=1000, k=5, input_dev=frames, scores_dev=scores,
                         tensor_dev=tensor)
    assert ws.run_noalloc(cfg, result, None) == ws.WS_OK
    torch.cuda.synchronize()
    assert (result.cpu().numpy()[1:10:2] >= 0).all()
    v, i = topk(np.zeros(1000, np.float32), 5)
    assert i.tolist() == result.cpu().numpy()[1:10:2].tolist()
