"""Oracle for detection decode + greedy NMS on a YOLO-style head.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed (yolo.cu README: the end-to-end pipeline passage, where
DFL decode and NMS run inside the graph; the "GPU-resident NMS" highlight,
a greedy suppression over candidates taken in score order; the embedding
example, up to 300 boxes returned in source-image coordinates):

  head   float32 [4*16 + nc][A]: for each anchor, four 16-bin DFL
         distributions (left, top, right, bottom distances, bin-major within
         a side) and then nc class probabilities.  Anchors are the cells of
         the stride-8, -16 and -32 grids over the network input, level by
         level, row-major within a level, each at its cell centre.
  1. per anchor, the best class (first maximum; NaN never wins) and its
     probability `conf`; the anchor is a candidate when conf > conf_thr;
  2. per candidate, each side's distance is the expectation of bin index
     under the softmax of its 16 logits; the box is
     (cx - l, cy - t, cx + r, cy + b) * stride in network-input pixels;
  3. candidates in order of conf descending, then anchor ascending; a
     candidate is kept unless an earlier kept box of the same class (of any
     class when agnostic) has IoU > iou_thr with it; at most max_det kept;
  4. each kept box is mapped back through the letterbox (or plain resize)
     to source pixels and clipped to the source image.

Two layers:
  * `*_exact` functions are the definitions in float64 (math.exp, exact
    rationals for IoU), used by the pins in tests/test_oracle_detect.py;
  * the decision path (`decode_candidates`, `iou32`, `nms`, `detect`) does
    the same arithmetic in IEEE binary32, one rounding per operation, in a
    fixed order.  A detection result is a set of integer decisions (which
    anchors pass, which boxes suppress which); taking them in the device's
    precision, with the same operations, makes the expected result exact.
    The exponential is computed by a published method, not the host
    library: Cody and Waite's two-constant reduction x = n ln2 + r, then
    e^r by its degree-7 Taylor polynomial in Horner form, then scaling by
    2^n (Cody & Waite, "Software Manual for the Elementary Functions",
    1980, the exp chapter).  Its accuracy is pinned against math.exp.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

REG_MAX = 16
STRIDES = (8, 16, 32)
F32 = np.float32


def _bits(u: int) -> np.float32:
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


LOG2E = _bits(0x3FB8AA3B)        # log2(e) rounded to binary32
LN2_HI = _bits(0x3F317200)       # ln 2 to 15 significant bits: n * LN2_HI is exact for |n| < 512
LN2_LO = _bits(0x35BFBE8E)       # ln 2 - LN2_HI rounded to binary32
EXP_FLOOR = F32(-80.0)           # e^-80 is still a normal binary32 number
TAYLOR = [F32(1) / F32(math.factorial(k)) for k in range(8)]   # 1/k! as binary32 quotients


# --------------------------------------------------------------------------
# anchors and mapping
# --------------------------------------------------------------------------
def anchors(net_w: int, net_h: int):
    """(cx, cy, stride) per anchor in head order, cell units, float64."""
    out = []
    for s in STRIDES:
        for gy in range(net_h // s):
            for gx in range(net_w // s):
                out.append((gx + 0.5, gy + 0.5, s))
    return out


def num_anchors(net_w: int, net_h: int) -> int:
    return sum((net_w // s) * (net_h // s) for s in STRIDES)


# --------------------------------------------------------------------------
# float64 definitions (pinned; used by tests only)
# --------------------------------------------------------------------------
def dfl_exact(logits) -> float:
    """Softmax expectation of bin index over one side's 16 logits, float64."""
    l = [float(v) for v in logits]
    m = max(l)
    e = [math.exp(v - m) for v in l]
    return sum(i * w for i, w in enumerate(e)) / sum(e)


def box_exact(head: np.ndarray, a: int, net_w: int, net_h: int):
    cx, cy, s = anchors(net_w, net_h)[a]
    d = [dfl_exact(head[side * REG_MAX:(side + 1) * REG_MAX, a]) for side in range(4)]
    return ((cx - d[0]) * s, (cy - d[1]) * s, (cx + d[2]) * s, (cy + d[3]) * s)


def iou_exact(a, b) -> Fraction:
    a = [Fraction(float(v)) for v in a]
    b = [Fraction(float(v)) for v in b]
    iw = max(Fraction(0), min(a[2], b[2]) - max(a[0], b[0]))
    ih = max(Fraction(0), min(a[3], b[3]) - max(a[1], b[1]))
    inter = iw * ih
    union = (a[2] - a[0]) * (a[3] - a[1]) + (b[2] - b[0]) * (b[3] - b[1]) - inter
    return inter / union if union > 0 else Fraction(0)


# --------------------------------------------------------------------------
# binary32 decision path
# --------------------------------------------------------------------------
def exp32(x):
    """e^x for x <= 0, elementwise over float32 (Cody-Waite + Taylor-7)."""
    x = np.maximum(np.asarray(x, dtype=F32), EXP_FLOOR)
    n = np.rint(x * LOG2E)
    r = (x - n * LN2_HI) - n * LN2_LO
    p = np.full_like(r, TAYLOR[7])
    for k in range(6, -1, -1):
        p = p * r + TAYLOR[k]
    return np.ldexp(p, n.astype(np.int32)).astype(F32)


def dfl32(logits: np.ndarray) -> np.ndarray:
    """Distance per column of a [16][m] float32 block: max, shifted exps,
    then the weight sum and the index-weighted sum accumulated bin 0..15 in
    order, then one division."""
    logits = np.asarray(logits, dtype=F32)
    m = logits[0].copy()
    for b in range(1, REG_MAX):
        m = np.maximum(m, logits[b])
    e = [exp32(logits[b] - m) for b in range(REG_MAX)]
    s = e[0].copy()
    num = np.zeros_like(s)
    for b in range(1, REG_MAX):
        s = s + e[b]
        num = num + F32(b) * e[b]
    return (num / s).astype(F32)


def best_class(probs: np.ndarray):
    """Per anchor: (first index of the maximum, its value); NaN never wins and
    an all-NaN column gives (0, -inf)."""
    probs = np.asarray(probs, dtype=F32)
    nc, a = probs.shape
    best = np.full(a, -np.inf, dtype=F32)
    cls = np.zeros(a, dtype=np.int64)
    for c in range(nc):
        better = probs[c] > best
        best = np.where(better, probs[c], best)
        cls = np.where(better, c, cls)
    return cls, best


def decode_candidates(head: np.ndarray, net_w: int, net_h: int, nc: int, conf_thr: float):
    """Candidates in rank order: list of (anchor, class, conf float32, box float32[4])
    in network-input pixels."""
    head = np.asarray(head, dtype=F32)
    A = num_anchors(net_w, net_h)
    assert head.shape == (4 * REG_MAX + nc, A), head.shape
    cls, conf = best_class(head[4 * REG_MAX:])
    cand = np.nonzero(conf > F32(conf_thr))[0]
    anc = anchors(net_w, net_h)
    cx = np.array([anc[a][0] for a in cand], dtype=F32)
    cy = np.array([anc[a][1] for a in cand], dtype=F32)
    st = np.array([anc[a][2] for a in cand], dtype=F32)
    d = [dfl32(head[side * REG_MAX:(side + 1) * REG_MAX][:, cand]) for side in range(4)]
    x1 = (cx - d[0]) * st
    y1 = (cy - d[1]) * st
    x2 = (cx + d[2]) * st
    y2 = (cy + d[3]) * st
    out = [(int(a), int(cls[a]), conf[a], np.array([x1[i], y1[i], x2[i], y2[i]], dtype=F32))
           for i, a in enumerate(cand)]
    out.sort(key=lambda c: (-float(c[2]), c[0]))
    return out


def iou32(a: np.ndarray, b: np.ndarray) -> np.float32:
    """IoU of two xyxy boxes in binary32: areas, clipped intersection sides,
    intersection, union = (area_a + area_b) - inter, one division."""
    area_a = (a[2] - a[0]) * (a[3] - a[1])
    area_b = (b[2] - b[0]) * (b[3] - b[1])
    iw = np.maximum(F32(0), np.minimum(a[2], b[2]) - np.maximum(a[0], b[0]))
    ih = np.maximum(F32(0), np.minimum(a[3], b[3]) - np.maximum(a[1], b[1]))
    inter = iw * ih
    union = (area_a + area_b) - inter
    with np.errstate(invalid="ignore", divide="ignore"):
        return F32(inter / union)


def nms(cands, iou_thr: float, max_det: int, agnostic: bool = False):
    """Greedy suppression over candidates already in rank order."""
    t = F32(iou_thr)
    kept = []
    for c in cands:
        if len(kept) == max_det:
            break
        if any((agnostic or k[1] == c[1]) and iou32(k[3], c[3]) > t for k in kept):
            continue
        kept.append(c)
    return kept


def map_to_source(box: np.ndarray, left: int, top: int, sx: np.float32, sy: np.float32,
                  src_w: int, src_h: int) -> np.ndarray:
    """Network-input pixels -> source pixels: subtract the region origin,
    scale by source/region size (binary32 of the float64 quotient), clip."""
    x1 = np.minimum(np.maximum((box[0] - F32(left)) * sx, F32(0)), F32(src_w))
    y1 = np.minimum(np.maximum((box[1] - F32(top)) * sy, F32(0)), F32(src_h))
    x2 = np.minimum(np.maximum((box[2] - F32(left)) * sx, F32(0)), F32(src_w))
    y2 = np.minimum(np.maximum((box[3] - F32(top)) * sy, F32(0)), F32(src_h))
    return np.array([x1, y1, x2, y2], dtype=F32)


def detect(head: np.ndarray, src_w: int, src_h: int, net_w: int, net_h: int, region,
           nc: int, conf_thr: float, iou_thr: float, max_det: int, agnostic: bool = False):
    """Full decode + NMS + mapping.  `region` = (left, top, w, h) of the image
    inside the network input.  Returns (boxes float32[n][4], scores float32[n],
    classes int32[n], number of candidates)."""
    left, top, rw, rh = region
    sx = F32(src_w / rw)
    sy = F32(src_h / rh)
    cands = decode_candidates(head, net_w, net_h, nc, conf_thr)
    kept = nms(cands, iou_thr, max_det, agnostic)
    boxes = np.array([map_to_source(k[3], left, top, sx, sy, src_w, src_h) for k in kept],
                     dtype=F32).reshape(-1, 4)
    scores = np.array([k[2] for k in kept], dtype=F32)
    classes = np.array([k[1] for k in kept], dtype=np.int32)
    return boxes, scores, classes, len(cands)
