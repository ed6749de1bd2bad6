"""Oracle for the fused preprocess: RGB8 HWC -> resample -> normalise -> FP32 NCHW.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed (WarpStream TRT article, fused-preprocess passage and its
dataflow figure): for every destination pixel, a centre-aligned source
coordinate; the four bilinear neighbours of each RGB channel; interpolation;
scaling from byte range to [0, 1]; subtraction of the channel mean and
division by the channel standard deviation; the result lands directly in the
destination channel plane (planar NCHW).  No intermediate resized or
normalised HWC image exists, and nothing is rounded to bytes in between.

Readings taken where the pages are silent (each listed in the design notes):
  * Centre-aligned coordinate = half-pixel centres, align_corners=false:
    src = (d + 1/2) * S / R - 1/2, clamped below at 0; the right-hand tap is
    clamped to the last source pixel.  Evaluated here in exact rationals.
  * Normalisation order: (p / 255 - mean) / std, in float64.
  * Letterbox (yolo.cu README: GPU letterbox of the raw frame; aspect
    preserved): r = min(Dw/W, Dh/H); region Rw = floor(W r + 1/2),
    Rh = floor(H r + 1/2); left = floor((Dw - Rw) / 2), top =
    floor((Dh - Rh) / 2); the source is resampled onto the region with the
    per-axis rule above (S onto R); every other cell holds the pad byte value
    normalised like a pixel.  The odd pad split and the round-half-up of a
    non-integer W r are parity unpinned (no workload reaches them).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def axis_taps(src: int, dst: int):
    """Exact sampling taps for one axis: (i0[], i1[], w[]) for d = 0..dst-1.

    src = (d + 1/2) * S / R - 1/2  ==  ((2d + 1) S - R) / (2R), clamped at 0.
    i0 = floor(src), w = src - i0 (exact fraction, then float64),
    i1 = min(i0 + 1, S - 1).
    """
    if src <= 0 or dst <= 0:
        raise ValueError("axis sizes must be positive")
    i0 = np.empty(dst, dtype=np.int64)
    i1 = np.empty(dst, dtype=np.int64)
    w = np.empty(dst, dtype=np.float64)
    for d in range(dst):
        pos = Fraction((2 * d + 1) * src - dst, 2 * dst)
        if pos < 0:
            pos = Fraction(0)
        lo = pos.numerator // pos.denominator
        i0[d] = lo
        i1[d] = min(lo + 1, src - 1)
        w[d] = float(pos - lo)
    return i0, i1, w


def letterbox_region(src_w: int, src_h: int, dst_w: int, dst_h: int):
    """(left, top, region_w, region_h) of the aspect-preserving letterbox box."""
    r = min(Fraction(dst_w, src_w), Fraction(dst_h, src_h))
    half = Fraction(1, 2)
    rw = int((src_w * r + half) // 1)
    rh = int((src_h * r + half) // 1)
    rw = max(1, min(rw, dst_w))
    rh = max(1, min(rh, dst_h))
    return (dst_w - rw) // 2, (dst_h - rh) // 2, rw, rh


def pad_value(pad: float, mean, std) -> np.ndarray:
    """Normalised value of a pad cell per channel: (pad/255 - mean) / std."""
    return np.array([(pad / 255.0 - mean[c]) / std[c] for c in range(3)], dtype=np.float64)


def preprocess(frame: np.ndarray, dst_w: int, dst_h: int, mean, std,
               letterbox: bool = False, pad: float = 114.0) -> np.ndarray:
    """One uint8 [H][W][3] RGB frame -> float64 [3][dst_h][dst_w]."""
    frame = np.asarray(frame)
    if frame.dtype != np.uint8 or frame.ndim != 3 or frame.shape[2] != 3:
        raise ValueError("frame must be uint8 [H][W][3]")
    h, w = frame.shape[0], frame.shape[1]
    if letterbox:
        left, top, rw, rh = letterbox_region(w, h, dst_w, dst_h)
    else:
        left, top, rw, rh = 0, 0, dst_w, dst_h

    x0, x1, wx = axis_taps(w, rw)
    y0, y1, wy = axis_taps(h, rh)
    p = frame.astype(np.float64)
    p00 = p[y0][:, x0]          # [rh][rw][3]
    p01 = p[y0][:, x1]
    p10 = p[y1][:, x0]
    p11 = p[y1][:, x1]
    ax = wx[None, :, None]
    ay = wy[:, None, None]
    top_row = (1.0 - ax) * p00 + ax * p01
    bot_row = (1.0 - ax) * p10 + ax * p11
    val = (1.0 - ay) * top_row + ay * bot_row          # [rh][rw][3], byte units

    out = np.empty((3, dst_h, dst_w), dtype=np.float64)
    padv = pad_value(pad, mean, std)
    for c in range(3):
        out[c, :, :] = padv[c]
        out[c, top:top + rh, left:left + rw] = (val[:, :, c] / 255.0 - mean[c]) / std[c]
    return out


def preprocess_batch(frames: np.ndarray, dst_w: int, dst_h: int, mean, std,
                     letterbox: bool = False, pad: float = 114.0) -> np.ndarray:
    """uint8 [B][H][W][3] -> float64 [B][3][dst_h][dst_w], frame by frame."""
    return np.stack([preprocess(f, dst_w, dst_h, mean, std, letterbox, pad) for f in frames])
