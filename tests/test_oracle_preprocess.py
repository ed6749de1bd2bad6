"""Pins for the preprocess oracle: closed forms, invariants, hand-worked cases and
a library cross-check, each independent of the oracle's own code.

Pinned facts (WarpStream TRT article, fused-preprocess passage; bilinear sampling
with half-pixel centres, align_corners=false, edge clamp; letterbox per the
yolo.cu README):
  * identity resize reduces to pure per-pixel normalisation with HWC->CHW;
  * a constant image gives constant planes (taps' weights sum to one);
  * hand-derived 1-D taps for 4->2, 2->4, 3->2, 1->3;
  * an exact factor-2 downscale is the 2x2 block mean;
  * general shapes match torch's float64 bilinear interpolate (align_corners=False);
  * a letterbox puts the pad value outside the region and the resampled frame inside.
"""
import itertools

import numpy as np
import pytest

from oracle import axis_taps, letterbox_region, pad_value, preprocess, preprocess_batch
from post_processing_amd import workloads as wl

MEAN = wl.IMAGENET_MEAN
STD = wl.IMAGENET_STD


def norm(v, c, mean=MEAN, std=STD):
    return (np.asarray(v, dtype=np.float64) / 255.0 - mean[c]) / std[c]


def one_row_frame(vals):
    """A 1-pixel-high frame whose R channel holds vals (G, B zero)."""
    f = np.zeros((1, len(vals), 3), dtype=np.uint8)
    f[0, :, 0] = vals
    return f


@pytest.mark.parametrize("src,dst,expected", [
    # taps derived by hand from src = (d + 1/2) S/R - 1/2, clamped at 0 / S-1
    (4, 2, [[0.5, 0.5, 0, 0], [0, 0, 0.5, 0.5]]),
    (2, 4, [[1, 0], [0.75, 0.25], [0.25, 0.75], [0, 1]]),
    (3, 2, [[0.75, 0.25, 0], [0, 0.25, 0.75]]),
    (1, 3, [[1], [1], [1]]),
    (5, 1, [[0, 0, 1, 0, 0]]),
    (6, 4, [[0.75, 0.25, 0, 0, 0, 0], [0, 0.25, 0.75, 0, 0, 0],
            [0, 0, 0, 0.75, 0.25, 0], [0, 0, 0, 0, 0.25, 0.75]]),
])
def test_hand_worked_axis(src, dst, expected):
    vals = np.array([17, 200, 3, 99, 150, 42][:src], dtype=np.uint8)
    out = preprocess(one_row_frame(vals), dst, 1, MEAN, STD)
    want = norm(np.asarray(expected, dtype=np.float64) @ vals.astype(np.float64), 0)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-12)
    # the same taps along y (transposed frame) -- catches swapped axes
    f = np.zeros((src, 1, 3), dtype=np.uint8)
    f[:, 0, 1] = vals
    out_y = preprocess(f, 1, dst, MEAN, STD)
    np.testing.assert_allclose(out_y[1, :, 0], norm(np.asarray(expected) @ vals.astype(float), 1),
                               rtol=0, atol=1e-12)


def test_axis_taps_exact_weights():
    # 1080 -> 224: src = (2d+1)*1080/448 - 1/2, check a few d by integer arithmetic
    i0, i1, w = axis_taps(1080, 224)
    for d in (0, 1, 7, 100, 223):
        num, den = (2 * d + 1) * 1080 - 224, 448
        assert i0[d] == num // den and w[d] == (num % den) / den
        assert i1[d] == min(num // den + 1, 1079)
    assert (np.diff(i0) >= 0).all() and (w >= 0).all() and (w < 1).all()


@pytest.mark.parametrize("h,w", [(5, 7), (1, 1), (3, 64), (48, 64)])
def test_identity_resize_is_normalisation(h, w):
    rng = np.random.default_rng(h * 100 + w)
    f = rng.integers(0, 256, size=(h, w, 3), dtype=np.uint8)
    out = preprocess(f, w, h, MEAN, STD)
    for c in range(3):
        np.testing.assert_allclose(out[c], norm(f[:, :, c], c), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(48, 64, 32, 32), (7, 5, 13, 11), (1, 9, 4, 1), (67, 1, 3, 67)])
def test_constant_image_gives_constant_planes(shape):
    h, w, dh, dw = shape
    f = np.empty((h, w, 3), dtype=np.uint8)
    f[..., 0], f[..., 1], f[..., 2] = 10, 128, 251       # distinct per channel: pins RGB order
    out = preprocess(f, dw, dh, MEAN, STD)
    for c, v in enumerate((10, 128, 251)):
        np.testing.assert_allclose(out[c], norm(v, c), rtol=0, atol=1e-12)


def test_factor_two_is_block_mean():
    rng = np.random.default_rng(5)
    f = rng.integers(0, 256, size=(18, 26, 3), dtype=np.uint8)
    out = preprocess(f, 13, 9, MEAN, STD)
    blk = f.astype(np.float64).reshape(9, 2, 13, 2, 3).mean(axis=(1, 3))
    for c in range(3):
        np.testing.assert_allclose(out[c], norm(blk[:, :, c], c), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_matches_torch_bilinear(seed):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(300 + seed)
    h, w, dh, dw = (int(v) for v in rng.integers(1, 70, size=4))
    f = rng.integers(0, 256, size=(h, w, 3), dtype=np.uint8)
    out = preprocess(f, dw, dh, (0.0, 0.0, 0.0), (1.0 / 255, 1.0 / 255, 1.0 / 255))  # byte units
    t = torch.from_numpy(f.astype(np.float64)).permute(2, 0, 1)[None]
    ref = F.interpolate(t, size=(dh, dw), mode="bilinear", align_corners=False,
                        antialias=False)[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-9)


def test_matches_torch_bilinear_c2_shape():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    w = wl.c2()
    out = preprocess(w.frames[0], 224, 224, (0.0, 0.0, 0.0), (1 / 255, 1 / 255, 1 / 255))
    t = torch.from_numpy(w.frames[0].astype(np.float64)).permute(2, 0, 1)[None]
    ref = F.interpolate(t, size=(224, 224), mode="bilinear", align_corners=False,
                        antialias=False)[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-9)


@pytest.mark.parametrize("src,dst,box", [
    ((1280, 720), (640, 640), (0, 140, 640, 360)),
    ((720, 1280), (640, 640), (140, 0, 360, 640)),
    ((64, 48), (64, 48), (0, 0, 64, 48)),
    ((100, 50), (50, 50), (0, 12, 50, 25)),
    ((3, 1), (8, 8), (0, 2, 8, 3)),      # W r = 8, H r = 8/3 -> round half up 3, top (8-3)//2
])
def test_letterbox_region(src, dst, box):
    assert letterbox_region(*src, *dst) == box


def test_letterbox_c3_layout():
    w = wl.c3()
    out = preprocess(w.frames[0], 640, 640, w.mean, w.std, letterbox=True, pad=w.pad)
    assert out.shape == (3, 640, 640)
    np.testing.assert_array_equal(out[:, :140, :], 114.0 / 255.0)
    np.testing.assert_array_equal(out[:, 500:, :], 114.0 / 255.0)
    # content: scale exactly 1/2 on both axes -> 2x2 block means of the frame
    blk = w.frames[0].astype(np.float64).reshape(360, 2, 640, 2, 3).mean(axis=(1, 3))
    np.testing.assert_allclose(out[:, 140:500, :], np.moveaxis(blk, 2, 0) / 255.0,
                               rtol=0, atol=1e-12)


def test_letterbox_pad_columns_and_value():
    rng = np.random.default_rng(9)
    f = rng.integers(0, 256, size=(40, 20, 3), dtype=np.uint8)      # portrait into square
    mean, std = (0.1, 0.2, 0.3), (0.5, 0.6, 0.7)
    out = preprocess(f, 30, 30, mean, std, letterbox=True, pad=7.0)
    left, top, rw, rh = letterbox_region(20, 40, 30, 30)
    assert (left, top, rw, rh) == (7, 0, 15, 30)
    for c in range(3):
        pv = (7.0 / 255.0 - mean[c]) / std[c]
        np.testing.assert_allclose(out[c, :, :left], pv, rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[c, :, left + rw:], pv, rtol=0, atol=1e-15)
    np.testing.assert_allclose(pad_value(7.0, mean, std),
                               [(7 / 255 - m) / s for m, s in zip(mean, std)], atol=1e-15)
    # inside: the same resample as a plain resize of the frame onto the region
    inner = preprocess(f, rw, rh, mean, std)
    np.testing.assert_allclose(out[:, top:top + rh, left:left + rw], inner, rtol=0, atol=1e-15)


def test_batch_is_per_frame():
    rng = np.random.default_rng(4)
    fs = rng.integers(0, 256, size=(3, 6, 10, 3), dtype=np.uint8)
    ob = preprocess_batch(fs, 4, 5, MEAN, STD)
    for i in range(3):
        np.testing.assert_array_equal(ob[i], preprocess(fs[i], 4, 5, MEAN, STD))


def test_output_range_bound():
    # |out| <= max over bytes and channels of |(b/255 - mean)/std| (convex combination)
    rng = np.random.default_rng(11)
    f = rng.integers(0, 256, size=(37, 53, 3), dtype=np.uint8)
    out = preprocess(f, 29, 31, MEAN, STD)
    bound = max(abs((b / 255 - MEAN[c]) / STD[c]) for b in (0, 255) for c in range(3))
    assert np.abs(out).max() <= bound + 1e-12
    assert np.isfinite(out).all()
