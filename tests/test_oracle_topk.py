"""Pins for the Top-K oracle, independent of its own code.

Pinned facts (WarpStream TRT article, Top-K passage): exact selection of the K
best score/index pairs, listed rank by rank; ties prefer the lower class index;
NaN counts as negative infinity.
  * an independent naive repeated-argmax (the rank-by-rank selection the
    article describes), written here with explicit comparisons;
  * numpy's stable lexsort as a library second opinion;
  * exhaustive permutations of small multisets with ties, NaN, +-0, +-inf;
  * selection invariants at the workloads' full sizes.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import topk
from post_processing_amd import workloads as wl


def better(a, ia, b, ib):
    """Is (value a, index ia) ranked before (b, ib)?  NaN -> -inf."""
    a = -math.inf if math.isnan(a) else a
    b = -math.inf if math.isnan(b) else b
    return a > b or (a == b and ia < ib)


def naive_repeated_argmax(s, k):
    chosen = []
    taken = set()
    for _ in range(k):
        best = None
        for i in range(len(s)):
            if i in taken:
                continue
            if best is None or better(float(s[i]), i, float(s[best]), best):
                best = i
        chosen.append(best)
        taken.add(best)
    return chosen


def reported_bits(s, idx):
    b = np.asarray(s, dtype=np.float32).view(np.uint32)[idx].copy()
    b[np.isnan(np.asarray(s, dtype=np.float32)[idx])] = 0xFF800000
    return b


def check(s, k):
    vals, idx = topk(s, k)
    want = naive_repeated_argmax(s, k)
    assert idx.tolist() == want
    np.testing.assert_array_equal(vals.view(np.uint32), reported_bits(s, np.asarray(want)))


@pytest.mark.parametrize("seed,n,k", [(0, 1, 1), (1, 2, 2), (2, 63, 5), (3, 64, 32), (4, 65, 32),
                                      (5, 200, 10), (6, 300, 1), (7, 129, 31)])
def test_vs_naive_repeated_argmax(seed, n, k):
    s = wl.scores_with_specials(seed, n, tie_frac=0.2, nan_frac=0.05)
    check(s, k)


def test_exhaustive_small_multisets():
    pool = [np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, 1.0, np.inf]
    for n in range(1, 6):
        for combo in itertools.combinations(range(len(pool)), n):
            base = [pool[i] for i in combo]
            for perm in set(itertools.permutations(range(n))):
                s = np.array([base[p] for p in perm], dtype=np.float32)
                for k in range(1, n + 1):
                    check(s, k)


def test_vs_numpy_lexsort():
    s = wl.scores_with_specials(42, 5000, tie_frac=0.3, nan_frac=0.01)
    key = np.where(np.isnan(s), -np.inf, s.astype(np.float64))
    order = np.lexsort((np.arange(s.size), -key))      # last key is primary
    vals, idx = topk(s, 32)
    np.testing.assert_array_equal(idx, order[:32])
    np.testing.assert_array_equal(vals.view(np.uint32), reported_bits(s, order[:32]))


def test_nan_reported_as_neg_inf_and_signed_zero_kept():
    s = np.array([np.nan, -0.0, 0.0, np.nan, -np.inf], dtype=np.float32)
    vals, idx = topk(s, 5)
    assert idx.tolist() == [1, 2, 0, 3, 4]        # -0 == +0 -> index; NaN == -inf -> index
    assert vals.view(np.uint32).tolist() == [0x80000000, 0x00000000, 0xFF800000, 0xFF800000,
                                              0xFF800000]


def test_subnormals_not_flushed():
    s = np.array([0.0, 1e-45, 1e-40, -1e-45], dtype=np.float32)
    vals, idx = topk(s, 4)
    assert idx.tolist() == [2, 1, 0, 3]


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        topk(np.zeros(3, np.float32), 0)
    with pytest.raises(ValueError):
        topk(np.zeros(3, np.float32), 4)


def invariants(s, k, vals, idx):
    key = np.where(np.isnan(s), -np.inf, s.astype(np.float64))
    assert len(set(idx.tolist())) == k
    kv = key[idx]
    assert (np.diff(kv) <= 0).all()
    for a in range(k - 1):
        if kv[a] == kv[a + 1]:
            assert idx[a] < idx[a + 1]
    rest = np.ones(s.size, dtype=bool)
    rest[idx] = False
    j = np.flatnonzero(rest)
    last_k, last_i = kv[-1], idx[-1]
    ok = (key[j] < last_k) | ((key[j] == last_k) & (j > last_i))
    assert ok.all()
    np.testing.assert_array_equal(vals.view(np.uint32), reported_bits(s, idx))


@pytest.mark.parametrize("cfg", ["c1", "c3", "c4"])
def test_invariants_full_size(cfg):
    w = wl.ALL_CONFIGS[cfg]()
    vals, idx = topk(w.scores, w.k)
    invariants(w.scores, w.k, vals, idx)


def test_planted_ties_reach_top_k():
    # C1 and C4 plant copies of their largest values: the top-K must contain tie pairs
    for cfg in ("c1", "c4"):
        w = wl.ALL_CONFIGS[cfg]()
        vals, idx = topk(w.scores, w.k)
        assert np.unique(vals).size < w.k
