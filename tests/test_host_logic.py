"""Host logic of the lane library, on the CPU (no GPU, no HIP calls).

* The planning code (csrc/ws_plan.h) is compiled with g++ into a small driver
  and its exact sampling taps and letterbox boxes are compared with the
  oracle's; its config validation and lane state machine are checked by the
  driver's self-test (misuse -> error codes).
* The built library loads and exports every function include/*.h declares.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import axis_taps, letterbox_region
from post_processing_amd import build as ppbuild


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host") / "ws_plan_test")
    return ppbuild.build_host_test(out)


def run(driver, *args):
    res = subprocess.run([driver, *map(str, args)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return res.stdout


def test_selftest(driver):
    out = run(driver, "selftest")
    assert "0 failures" in out


@pytest.mark.parametrize("S,R", [(1080, 224), (1920, 224), (720, 360), (1280, 640), (48, 32),
                                 (64, 32), (2160, 384), (3840, 384), (720, 224), (1280, 224),
                                 (2, 4), (1, 7), (7, 1), (67, 3), (3, 67), (16384, 1)])
def test_taps_match_oracle(driver, S, R):
    rows = [line.split() for line in run(driver, "taps", S, R).splitlines()]
    i0, i1, w = axis_taps(S, R)
    assert [int(r[0]) for r in rows] == i0.tolist()
    assert [int(r[1]) for r in rows] == i1.tolist()
    gw = np.array([float(r[2]) for r in rows]).astype(np.float32)   # %.9g round-trips FP32
    np.testing.assert_allclose(gw, w.astype(np.float32), rtol=0, atol=0)


@pytest.mark.parametrize("src,dst", [((1280, 720), (640, 640)), ((720, 1280), (640, 640)),
                                     ((100, 50), (50, 50)), ((3, 1), (8, 8)), ((1, 67), (1, 1)),
                                     ((20, 40), (30, 30)), ((641, 479), (640, 640)),
                                     ((1920, 1080), (640, 384)), ((5, 5), (3, 9))])
def test_letterbox_matches_oracle(driver, src, dst):
    got = tuple(int(v) for v in run(driver, "letterbox", *src, *dst).split())
    assert got == letterbox_region(*src, *dst)


def test_library_exports_declared_symbols():
    from post_processing_amd import ws
    if not os.path.exists(ws.LIB_PATH):
        ppbuild.build_lib()
    lib = ws.load()
    names = ws.declared_functions()
    assert {"ws_create_lane", "ws_submit", "ws_wait", "ws_destroy"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_config_struct_layout():
    # LaneConfig must match the C layout (x86-64 SysV): doubles 8-aligned,
    # pointers after the int32 fields, 136 bytes total.
    import ctypes
    from post_processing_amd import ws
    assert ctypes.sizeof(ws.LaneConfig) == 152
    assert ws.LaneConfig.pad_value.offset == 32
    assert ws.LaneConfig.input_dev.offset == 104
    assert ctypes.sizeof(ws.TopkEntry) == 8
    assert ctypes.sizeof(ws.LaneView) == 56
