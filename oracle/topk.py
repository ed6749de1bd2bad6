"""Oracle for the exact Top-K over FP32 scores.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed (WarpStream TRT article, Top-K passage): the K best
score/index pairs of a fixed-size FP32 vector, K <= 32, ranked by score
descending; equal scores prefer the lower class index; NaN is treated as
negative infinity.  The result is listed rank by rank.

Written as the plain definition: a full stable sort by (-key, index), where
key = -inf for NaN and the IEEE value otherwise (so -0.0 and +0.0 compare
equal and the index decides).  Readings: a NaN's reported value is -inf
(bits 0xFF800000); any other selected value is reported with its original
bits (so -0.0 stays -0.0, and subnormals are compared and kept unflushed).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF_BITS = 0xFF800000


def topk_keys_order(scores: np.ndarray):
    """Indices of all N scores in rank order (full stable sort)."""
    s = np.asarray(scores, dtype=np.float32)
    keys = [(-math.inf if math.isnan(v) else v) for v in s.astype(np.float64).tolist()]
    return sorted(range(len(keys)), key=lambda i: (-keys[i], i))


def topk(scores: np.ndarray, k: int):
    """Top-k of float32 scores -> (values float32[k], indices int32[k]).

    Values keep their original bit pattern except NaN, reported as -inf.
    """
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[0]
    if not (1 <= k <= n):
        raise ValueError(f"k={k} out of range for n={n}")
    order = topk_keys_order(s)[:k]
    bits = s.view(np.uint32)[order].copy()
    nan = np.isnan(s[order])
    bits[nan] = NEG_INF_BITS
    return bits.view(np.float32), np.asarray(order, dtype=np.int32)
