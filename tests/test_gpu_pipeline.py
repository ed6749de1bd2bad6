"""GPU parity of the lane pipeline against the CPU oracle, through the C ABI.

Bar: the FP32 tensor within 1e-5 absolute of the float64 oracle everywhere;
Top-K indices and value bits identical.  Every workload is run in the launch
configuration the benchmark uses (captured graph, automatic geometry).
"""
import os

import numpy as np
import pytest

from oracle import preprocess_batch, topk
from post_processing_amd import workloads as wl
from post_processing_amd import ws

from gpu_util import (Run, assert_rounded_close, assert_tensor_close, assert_topk_exact,
                      oracle_outputs)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_parity_device_input(gpu_lib, name):
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    r = Run(w, host_input=False)
    try:
        r.run()
        t, tk = r.outputs()
        err = assert_tensor_close(t, ref)
        assert_topk_exact(tk, rtk)
        print(f"{name}: max|err| {err:.2e}, plan {r.lane.plan()}")
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_parity_mapped_host_input(gpu_lib, name):
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    r = Run(w, host_input=True)
    try:
        r.run()
        t, tk = r.outputs()
        assert_tensor_close(t, ref)
        assert_topk_exact(tk, rtk)
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_parity_copy_input(gpu_lib, name):
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    r = Run(w, input_mode=ws.INPUT_COPY)
    try:
        assert r.lane.plan()["graph_nodes"] == 3
        r.run()
        t, tk = r.outputs()
        assert_tensor_close(t, ref)
        assert_topk_exact(tk, rtk)
    finally:
        r.close()


def test_input_modes_agree_bitwise(gpu_lib):
    w = wl.c2()
    runs = [Run(w, input_mode=m) for m in (ws.INPUT_DEVICE, ws.INPUT_MAPPED_HOST, ws.INPUT_COPY)]
    try:
        outs = []
        for r in runs:
            r.run()
            outs.append(r.outputs())
        for t, tk in outs[1:]:
            np.testing.assert_array_equal(t.view(np.uint32), outs[0][0].view(np.uint32))
            assert_topk_exact(tk, outs[0][1])
    finally:
        for r in runs:
            r.close()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_reduced_precision_tensor(gpu_lib, name, fmt):
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    dt = ws.DTYPE_F16 if fmt == "f16" else ws.DTYPE_BF16
    r = Run(w, host_input=False, tensor_dtype=dt)
    try:
        r.run()
        t, tk = r.outputs()
        worst = assert_rounded_close(t, ref, fmt)
        assert_topk_exact(tk, rtk)
        print(f"{name} {fmt}: worst error {worst:.3f} ulp")
    finally:
        r.close()


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_reduced_precision_small_shapes(gpu_lib, seed, fmt):
    w = wl.random_small(100 + seed, letterbox=bool(seed % 2))
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=False, tensor_dtype=ws.DTYPE_F16 if fmt == "f16" else ws.DTYPE_BF16,
            pixels_per_thread=(1, 2, 4)[seed % 3])
    try:
        r.run()
        assert_rounded_close(r.outputs()[0], ref, fmt)
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_bgr_input(gpu_lib, name):
    # A BGR producer's frame is the RGB frame with its channel axis reversed;
    # the BGR lane must give the RGB lane's tensor bit for bit, and the oracle's.
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    bgr = wl.Workload(w.name + "_bgr", w.src_w, w.src_h, w.dst_w, w.dst_h, w.mode, w.mean, w.std,
                      w.pad, w.k, np.ascontiguousarray(w.frames[..., ::-1]), w.scores)
    a = Run(w, host_input=False)
    b = Run(bgr, host_input=False, channel_order=ws.CHANNELS_BGR)
    try:
        a.run()
        b.run()
        ta, _ = a.outputs()
        tb, tk = b.outputs()
        np.testing.assert_array_equal(ta.view(np.uint32), tb.view(np.uint32))
        assert_tensor_close(tb, ref)
        assert_topk_exact(tk, rtk)
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("mode", ["device", "mapped"])
def test_throughput_batch_parity(gpu_lib, mode):
    """The 64-frame batch, from device memory (the bandwidth workload) and
    read over the bus from mapped pinned host memory."""
    w = wl.c5_throughput(64)
    ref, _ = oracle_outputs(w)
    r = Run(w, input_mode=ws.INPUT_DEVICE if mode == "device" else ws.INPUT_MAPPED_HOST)
    try:
        r.run()
        t, _ = r.outputs()
        assert_tensor_close(t, ref)
    finally:
        r.close()


@pytest.mark.parametrize("name,policy,dtype", [
    ("c2", "stream", ws.DTYPE_F32), ("c3", "stream", ws.DTYPE_F32), ("c4", "stream", ws.DTYPE_F32),
    ("c2", "stream", ws.DTYPE_F16), ("c3", "stream", ws.DTYPE_BF16), ("c5t", "keep", ws.DTYPE_F32)])
def test_cache_policies(gpu_lib, name, policy, dtype):
    """Both cache policies of the gather kernel (ordinary or non-temporal frame
    loads and tensor stores), each on workloads its automatic choice does not
    give it (single frames stream here, the 64-frame batch keeps), match the
    oracle and the other policy bit for bit; the lane reports the policy it
    runs."""
    w = wl.c5_throughput(64) if name == "c5t" else wl.ALL_CONFIGS[name]()
    ref, _ = oracle_outputs(w)
    mode = ws.CACHE_STREAM if policy == "stream" else ws.CACHE_KEEP
    r = Run(w, host_input=False, tensor_dtype=dtype, cache_policy=mode)
    a = Run(w, host_input=False, tensor_dtype=dtype)
    try:
        assert r.lane.plan()["streaming"] == (1 if policy == "stream" else 0)
        assert a.lane.plan()["streaming"] == (1 if name == "c5t" else 0)
        r.run()
        a.run()
        t, _ = r.outputs()
        u, _ = a.outputs()
        if dtype == ws.DTYPE_F32:
            assert_tensor_close(t, ref)
        else:
            assert_rounded_close(t, ref, "f16" if dtype == ws.DTYPE_F16 else "bf16")
        assert np.array_equal(t.view(np.uint32), u.view(np.uint32))
    finally:
        r.close()
        a.close()


@pytest.mark.parametrize("seed", range(24))
@pytest.mark.parametrize("letterbox", [False, True])
def test_random_small_shapes(gpu_lib, seed, letterbox):
    w = wl.random_small(seed, letterbox=letterbox)
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=bool(seed % 2), pixels_per_thread=(1, 2, 4)[seed % 3])
    try:
        r.run()
        t, _ = r.outputs()
        assert_tensor_close(t, ref)
    finally:
        r.close()


@pytest.mark.parametrize("sw,sh,dw,dh", [(1, 1, 5, 3), (2, 1, 7, 2), (3, 5, 9, 11), (5, 2, 5, 2),
                                         (7, 3, 13, 8)])
@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("host", [False, True])
def test_gather_windows_at_the_end_of_the_input(gpu_lib, sw, sh, dw, dh, batch, host):
    """Tiny frames upscaled (or copied) with one column per thread: the last
    output pixels tap the input's final bytes, whose 12-byte window would run
    past the end of the input and is read bytewise instead."""
    rng = np.random.default_rng(sw * 1000 + sh * 100 + dw * 10 + dh + batch)
    frames = rng.integers(0, 256, size=(batch, sh, sw, 3), dtype=np.uint8)
    w = wl.Workload(f"tail_{sw}x{sh}_to_{dw}x{dh}_b{batch}", sw, sh, dw, dh, wl.RESIZE,
                    (0.485, 0.456, 0.406), (0.229, 0.224, 0.225), 114.0, 0, frames, None)
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=host, pixels_per_thread=1)
    try:
        r.run()
        t, _ = r.outputs()
        assert_tensor_close(t, ref)
    finally:
        r.close()


@pytest.mark.parametrize("name,rows,px", [("c4", 1, 4), ("c4", 2, 1), ("c4", 3, 2), ("c4", 6, 4),
                                          ("c1", 5, 1), ("c1", 32, 2), ("c2", 9, 4), ("c2", 1, 2),
                                          ("c3", 4, 4), ("c3", 1, 1), ("c3", 2, 2)])
def test_launch_geometry_does_not_change_results(gpu_lib, name, rows, px):
    w = wl.ALL_CONFIGS[name]()
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=False, rows_per_group=rows, pixels_per_thread=px)
    try:
        assert r.lane.plan()["rows_per_group"] == rows
        r.run()
        t, _ = r.outputs()
        assert_tensor_close(t, ref)
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_autotuned_lane_matches_default_lane(gpu_lib, name):
    # The autotuner only picks launch geometry: its lane must reproduce the
    # default lane bit for bit, and the oracle to the usual bound.
    w = wl.ALL_CONFIGS[name]()
    ref, rtk = oracle_outputs(w)
    a = Run(w, host_input=False)
    b = Run(w, host_input=False, autotune=True)
    try:
        plan = b.lane.plan()
        assert plan["pixels_per_thread"] in (1, 2, 4)
        assert plan["rows_per_group"] in (1, 2, 4)
        for _ in range(2):
            a.run()
            b.run()
            ta, tka = a.outputs()
            tb, tkb = b.outputs()
            np.testing.assert_array_equal(ta.view(np.uint32), tb.view(np.uint32))
            assert_tensor_close(tb, ref)
            if w.k:
                assert_topk_exact(tkb, rtk)
                assert_topk_exact(tka, rtk)
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("px", [2, 4])
def test_rows_per_group_beyond_lds_rejected(gpu_lib, px):
    # 7 staged row pairs of 3840-pixel rows need ~161 KB of LDS: more than a
    # workgroup may hold, so a staged lane refuses the plan instead of
    # launching it.
    with pytest.raises(ws.WsError) as ei:
        Run(wl.c4(), host_input=False, rows_per_group=7, pixels_per_thread=px)
    assert ei.value.status == ws.WS_E_INVALID_ARG


def test_gather_kernel_takes_rows_the_staged_kernel_cannot(gpu_lib):
    # The gather kernel (one column per thread) stages nothing, so the same
    # seven rows per workgroup are accepted, allocate no LDS, and match the
    # oracle.
    w = wl.c4()
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=False, rows_per_group=7, pixels_per_thread=1)
    try:
        plan = r.lane.plan()
        assert plan["rows_per_group"] == 7 and plan["pre_lds_bytes"] == 0
        r.run()
        assert_tensor_close(r.outputs()[0], ref)
    finally:
        r.close()


def _topk_workload(n, k, seed):
    s = wl.scores_with_specials(seed, n, tie_frac=0.2, nan_frac=0.02)
    frame = np.zeros((1, 4, 4, 3), dtype=np.uint8)
    return wl.Workload(f"topk_{n}_{k}", 4, 4, 4, 4, wl.RESIZE, (0, 0, 0), (1, 1, 1), 114.0, k,
                       frame, s)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 1000, 4096, 4097, 8192, 8193, 65537, 196608,
                               196609, 672000])
@pytest.mark.parametrize("k", [1, 5, 10, 31, 32])
def test_topk_edge_sizes(gpu_lib, n, k):
    """Sizes at the planner's boundaries too: one workgroup of one batch per
    wave up to 4 Ki scores, of 32 per lane up to 8 Ki, then 4 Ki chunks, and
    8 Ki chunks past 192 Ki."""
    if k > n:
        pytest.skip("K > N is rejected at create")
    w = _topk_workload(n, k, seed=n * 37 + k)
    rtk = topk(w.scores, k)
    r = Run(w, host_input=False)
    try:
        r.run()
        _, tk = r.outputs()
        assert_topk_exact(tk, rtk)
    finally:
        r.close()


@pytest.mark.parametrize("groups", [2, 13, 24, 50, 83, 128, 129])
@pytest.mark.parametrize("k", [7, 32])
def test_topk_merge_sizes(gpu_lib, groups, k):
    """1 Ki-score workgroups, so `groups` lists are published (the last one
    ragged): the fold merge at each register count it is built for (1, 2, 4,
    8, 12 and 16 per wave: 2 .. 128 lists) and the bound merge past 128."""
    n = groups * 1024 - 5
    w = _topk_workload(n, k, seed=groups * 101 + k)
    r = Run(w, host_input=False, topk_chunk=1024)
    try:
        assert r.lane.plan()["topk_groups"] == groups
        r.run()
        _, tk = r.outputs()
        assert_topk_exact(tk, topk(w.scores, k))
    finally:
        r.close()


@pytest.mark.parametrize("chunk", [1024, 2048, 8192, 65536, 688128])
def test_topk_chunking_does_not_change_results(gpu_lib, chunk):
    w = wl.c3()
    rtk = topk(w.scores, w.k)
    r = Run(w, host_input=False, topk_chunk=chunk)
    try:
        r.run()
        _, tk = r.outputs()
        assert_topk_exact(tk, rtk)
    finally:
        r.close()


@pytest.mark.parametrize("period,chunk", [(8192, 8192), (1000, 8192), (1024, 1024), (3, 4096)])
def test_topk_every_workgroup_alike(gpu_lib, period, chunk):
    """Scores repeating with a short period: every workgroup's K best have
    the same values, so nearly all published keys clear the bound and the
    merge selects among many survivors (with 1 Ki chunks, over several rounds
    of published keys)."""
    rng = np.random.default_rng(period * 7 + chunk)
    base = rng.normal(0.0, 1.0, period).astype(np.float32)
    s = np.tile(base, 700_000 // period + 1)[:700_000]
    frame = np.zeros((1, 4, 4, 3), dtype=np.uint8)
    w = wl.Workload("periodic", 4, 4, 4, 4, wl.RESIZE, (0, 0, 0), (1, 1, 1), 114.0, 32, frame, s)
    r = Run(w, host_input=False, topk_chunk=chunk)
    try:
        assert r.lane.plan()["topk_groups"] > 1
        r.run()
        _, tk = r.outputs()
        assert_topk_exact(tk, topk(s, 32))
    finally:
        r.close()


@pytest.mark.parametrize("n", [3000, 300_000])
def test_topk_all_equal_and_all_nan(gpu_lib, n):
    """Ties everywhere; NaN reported as -inf; both zeros keep their own sign
    bit in the result (3000 scores: one workgroup; 300,000: the merge)."""
    for vals in (np.full(n, 0.5, np.float32), np.full(n, np.nan, np.float32),
                 np.where(np.arange(n) % 2 == 0, 0.0, -0.0).astype(np.float32)):
        frame = np.zeros((1, 4, 4, 3), dtype=np.uint8)
        w = wl.Workload("same", 4, 4, 4, 4, wl.RESIZE, (0, 0, 0), (1, 1, 1), 114.0, 32, frame,
                        vals)
        r = Run(w, host_input=False)
        try:
            r.run()
            _, tk = r.outputs()
            assert_topk_exact(tk, topk(vals, 32))
        finally:
            r.close()


def test_replays_are_bitwise_stable(gpu_lib):
    w = wl.c2()
    r = Run(w, host_input=False)
    try:
        r.run()
        t0, tk0 = r.outputs()
        ms, wall = r.lane.bench(2000)
        assert (ms > 0).all()
        t1, tk1 = r.outputs()
        np.testing.assert_array_equal(t0.view(np.uint32), t1.view(np.uint32))
        assert_topk_exact(tk1, tk0)
    finally:
        r.close()


def test_graph_and_direct_launch_agree(gpu_lib):
    w = wl.c3()
    a = Run(w, host_input=False, use_graph=True)
    b = Run(w, host_input=False, use_graph=False)
    try:
        a.run()
        b.run()
        ta, ka = a.outputs()
        tb, kb = b.outputs()
        np.testing.assert_array_equal(ta.view(np.uint32), tb.view(np.uint32))
        assert_topk_exact(ka, kb)
    finally:
        a.close()
        b.close()


def test_mapped_and_device_input_agree(gpu_lib):
    w = wl.c2()
    a = Run(w, host_input=True)
    b = Run(w, host_input=False)
    try:
        a.run()
        b.run()
        np.testing.assert_array_equal(a.outputs()[0].view(np.uint32),
                                      b.outputs()[0].view(np.uint32))
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("mode", ["mapped", "copy"])
def test_host_slot_sees_each_new_frame(gpu_lib, mode):
    # The producer rewrites the slot between frames; every replay must read
    # the new bytes (no stale cached copy of the previous frame).
    w = wl.c1()
    r = Run(w, input_mode=ws.INPUT_MAPPED_HOST if mode == "mapped" else ws.INPUT_COPY)
    try:
        slot = r.lane.input_host_array()
        for i in range(4):
            frame = np.random.default_rng(500 + i).integers(0, 256, size=w.frames.shape,
                                                            dtype=np.uint8)
            slot[...] = frame
            r.run()
            ref = preprocess_batch(frame, w.dst_w, w.dst_h, w.mean, w.std)
            assert_tensor_close(r.outputs()[0], ref)
    finally:
        r.close()


POISON = np.uint32(0x7FC0DEAD)   # a NaN pattern no replay writes


@pytest.mark.parametrize("n,chunk,lists", [(1000, 0, 1), (65537, 0, 17), (672000, 0, 83),
                                           (129 * 1024 - 5, 1024, 129)])
def test_topk_scores_rewritten_between_replays(gpu_lib, n, chunk, lists):
    """New scores before every replay, with the result slot overwritten by a
    marker first, through the one-workgroup path, the fold merge (17 and 83
    lists) and the bound merge (129 lists).  A merge that read a previous
    launch's partial lists, or a replay that wrote nothing, would leave a
    stale or marked answer."""
    import torch
    w = _topk_workload(n, 32, seed=n + 3)
    r = Run(w, host_input=False, topk_chunk=chunk)
    try:
        assert r.lane.plan()["topk_groups"] == lists
        slot = r.lane.result_slot_words()
        for i in range(4):
            s = wl.scores_with_specials(700 + 13 * i + n % 97, n, tie_frac=0.2, nan_frac=0.01)
            if i % 2:
                s = -s          # a different order of magnitude of winners
            r.scores.copy_(torch.from_numpy(s))
            torch.cuda.synchronize()
            slot[:] = POISON
            r.run()
            assert not (slot == POISON).any()
            assert_topk_exact(r.outputs()[1], topk(s, 32))
    finally:
        r.close()


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_device_frame_rewritten_between_replays(gpu_lib, name):
    """A new frame in the borrowed device input and a poisoned tensor before
    every replay: each replay must produce the new frame's tensor."""
    import torch
    w = wl.ALL_CONFIGS[name]()
    r = Run(w, host_input=False)
    try:
        for i in range(3):
            frame = np.random.default_rng(800 + i).integers(0, 256, size=w.frames.shape,
                                                            dtype=np.uint8)
            r.frames.copy_(torch.from_numpy(frame))
            r.tensor.fill_(float("nan"))
            torch.cuda.synchronize()
            r.run()
            ref = preprocess_batch(frame, w.dst_w, w.dst_h, w.mean, w.std,
                                   letterbox=(w.mode == wl.LETTERBOX), pad=w.pad)
            assert_tensor_close(r.outputs()[0], ref)
    finally:
        r.close()


def test_topk_lanes_created_and_destroyed_back_to_back(gpu_lib):
    """Lanes of 65,537 scores, K = 10, created, run once and destroyed one
    after another, each on different scores: freed device buffers (partial
    lists, result slot) come back at the same addresses, so a read that
    returned a previous lane's data there would give a wrong answer."""
    import torch
    for i in range(8):
        s = wl.scores_with_specials(900 + i, 65537, tie_frac=0.2, nan_frac=0.02)
        frame = np.zeros((1, 4, 4, 3), dtype=np.uint8)
        w = wl.Workload("reuse", 4, 4, 4, 4, wl.RESIZE, (0, 0, 0), (1, 1, 1), 114.0, 10, frame, s)
        r = Run(w, host_input=False)
        try:
            slot = r.lane.result_slot_words()
            slot[:] = POISON
            r.run()
            assert_topk_exact(r.outputs()[1], topk(s, 10))
        finally:
            r.close()
            del r
            torch.cuda.synchronize()


def test_scores_rewritten_between_frames(gpu_lib):
    import torch
    w = wl.c1()
    r = Run(w, host_input=False)
    try:
        for i in range(3):
            s = wl.scores_with_specials(900 + i, w.num_scores, tie_frac=0.3)
            r.scores.copy_(torch.from_numpy(s))
            torch.cuda.synchronize()
            r.run()
            assert_topk_exact(r.outputs()[1], topk(s, w.k))
    finally:
        r.close()


def test_state_machine_misuse(gpu_lib):
    w = wl.c1()
    r = Run(w, host_input=False)
    lane = r.lane
    try:
        rc, _ = lane.wait()
        assert rc == ws.WS_E_STATE                   # nothing in flight
        assert lane.submit() == ws.WS_OK
        assert lane.submit() == ws.WS_E_STATE        # busy lane: no hidden queue
        rc, ms = lane.wait()
        assert rc == ws.WS_OK and ms > 0
        rc, _ = lane.wait()
        assert rc == ws.WS_E_STATE
        assert lane.submit() == ws.WS_OK             # destroy while in flight waits first
    finally:
        r.close()


def test_invalid_configs_rejected(gpu_lib):
    bad = [dict(k=33, num_scores=1000), dict(k=6, num_scores=5), dict(batch=0),
           dict(batch=65), dict(std=(0.2, 0.0, 0.2)), dict(pad=300.0), dict(src_w=0)]
    for b in bad:
        args = dict(src_w=64, src_h=48, dst_w=32, dst_h=32, mean=(0.4, 0.4, 0.4),
                    std=(0.2, 0.2, 0.2), num_scores=0, k=0)
        args.update(b)
        with pytest.raises(ws.WsError) as ei:
            ws.Lane(ws.make_config(**args))
        assert ei.value.status == ws.WS_E_INVALID_ARG


def test_eight_lanes_concurrently(gpu_lib):
    lanes = [wl.c5_lane(i) for i in range(8)]
    runs = [Run(w) for w in lanes]
    try:
        ms, wall = ws.bench_lanes([r.lane for r in runs], 50)
        assert ms.shape == (8, 50) and (ms > 0).all()
        for w, r in zip(lanes, runs):
            ref, rtk = oracle_outputs(w)
            t, tk = r.outputs()
            assert_tensor_close(t, ref)
            assert_topk_exact(tk, rtk)
    finally:
        for r in runs:
            r.close()


def test_library_loaded_before_torch_in_a_fresh_process(gpu_lib):
    """Loading the binding before PyTorch must still leave one HIP runtime in
    the process (the binding loads PyTorch first), so a lane can be created."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "from post_processing_amd import ws, workloads as wl\n"
        "ws.load()\n"
        "import torch\n"
        "maps = [l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l]\n"
        "assert len(set(maps)) == 1, sorted(set(maps))\n"
        "w = wl.c1()\n"
        "cfg = ws.make_config(src_w=w.src_w, src_h=w.src_h, dst_w=w.dst_w, dst_h=w.dst_h)\n"
        "with ws.Lane(cfg) as lane:\n"
        "    lane.run()\n"
        "print('ok')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=110)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stderr[-2000:]


def test_polled_signals_in_a_fresh_process(gpu_lib):
    """The deployment setting the benchmark uses: completion signals polled
    (HSA_ENABLE_INTERRUPT=0 before the HIP runtime starts).  In a fresh
    process, C2 and C3 lanes (C3's Top-K through the merge kernel) replay 300
    times and still match the oracle, and the launch-cost harness runs both
    of its forms."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import os, sys\n"
        "sys.path.insert(0, 'tests')\n"
        "assert os.environ.get('HSA_ENABLE_INTERRUPT') == '0'\n"
        "import torch\n"
        "from post_processing_amd import ws, workloads as wl\n"
        "from gpu_util import Run, oracle_outputs, assert_tensor_close, assert_topk_exact\n"
        "for name in ('c2', 'c3'):\n"
        "    w = wl.ALL_CONFIGS[name]()\n"
        "    ref, rtk = oracle_outputs(w)\n"
        "    r = Run(w, host_input=False)\n"
        "    try:\n"
        "        ms = r.lane.bench(300)[0]\n"
        "        assert (ms > 0).all()\n"
        "        r.run()\n"
        "        t, tk = r.outputs()\n"
        "        assert_tensor_close(t, ref)\n"
        "        assert_topk_exact(tk, rtk)\n"
        "    finally:\n"
        "        r.close()\n"
        "for form in (ws.LAUNCH_GRAPH, ws.LAUNCH_DIRECT):\n"
        "    c = ws.launch_cost(2, form, replays=50, warmup=10)\n"
        "    assert all((a > 0).all() for a in c.values()), (form, c)\n"
        "print('ok')\n")
    env = dict(os.environ, HSA_ENABLE_INTERRUPT="0")
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=110, env=env)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stderr[-2000:]


@pytest.mark.parametrize("shape", [(16384, 6, 16384, 3, False), (5, 16384, 3, 16384, False),
                                   (16384, 64, 4096, 64, True)])
def test_maximum_sides(gpu_lib, shape):
    """Frames and tensors at the 16384-pixel side limit: the widest rows
    (49,152 bytes each, two staged per output row) and the tallest columns."""
    sw, sh, dw, dh, letterbox = shape
    rng = np.random.default_rng(sw + 7 * sh + dw)
    frames = rng.integers(0, 256, size=(1, sh, sw, 3), dtype=np.uint8)
    w = wl.Workload(f"max_side_{sw}x{sh}_to_{dw}x{dh}", sw, sh, dw, dh,
                    wl.LETTERBOX if letterbox else wl.RESIZE, wl.IMAGENET_MEAN, wl.IMAGENET_STD,
                    114.0, 0, frames, None)
    ref, _ = oracle_outputs(w)
    r = Run(w, host_input=False)
    try:
        r.run()
        t, _ = r.outputs()
        assert_tensor_close(t, ref)
    finally:
        r.close()


def _order_keys(s):
    """(value descending, index ascending) as distinct uint64 keys: NaN ranks as
    -inf and -0 as +0; larger key = better."""
    b = s.view(np.uint32).copy()
    b[(b & 0x7FFFFFFF) > 0x7F800000] = 0xFF800000
    b[b == 0x80000000] = 0
    img = np.where(b >> 31 == 1, ~b, b | np.uint32(0x80000000)).astype(np.uint64)
    idx = np.arange(s.size, dtype=np.uint64)
    return (img << np.uint64(32)) | (~idx & np.uint64(0xFFFFFFFF))


@pytest.mark.parametrize("k", [1, 32])
def test_topk_four_million_scores(gpu_lib, k):
    """2^22 scores with ties, NaN and specials: checked by the properties that
    define the exact top K at any size (distinct keys, descending, and no
    unselected key above the K-th), then ordered by the oracle on the selected
    set."""
    n = 1 << 22
    w = _topk_workload(n, k, 77)
    r = Run(w, host_input=False)
    try:
        r.run()
        gv, gi = r.outputs()[1]
    finally:
        r.close()
    keys = _order_keys(w.scores)
    assert len(set(gi.tolist())) == k and (gi >= 0).all() and (gi < n).all()
    sel = keys[gi]
    assert (sel[:-1] > sel[1:]).all()            # strictly descending (integer keys)
    mask = np.ones(n, dtype=bool)
    mask[gi] = False
    assert keys[mask].max() < sel[-1]
    sub_v, sub_i = topk(w.scores[gi], k)          # the oracle on the selected set
    np.testing.assert_array_equal(gi[sub_i], gi)
    np.testing.assert_array_equal(gv.view(np.uint32), sub_v.view(np.uint32))
