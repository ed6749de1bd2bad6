"""Detection results checked against the float64 definitions, with derived
bounds for everything binary32 arithmetic may change.

The detection stage (yolo.cu README: DFL decode and greedy NMS inside the
graph; boxes returned in source-image coordinates) decides in binary32.  The
oracle's decision path repeats those operations bit for bit; this module
instead ties a result -- from the GPU or from that decision path -- to the
plain float64 definitions in oracle/detect.py (`dfl_exact`, `box_exact`'s
formula, `iou_exact`), so that a shared mistake of the binary32 layer and the
kernel cannot hide.

What is exact and what is bounded (u = 2^-24, the binary32 unit roundoff):
  * Candidates, best class and rank order compare binary32 inputs only (the
    head's probabilities and the binary32 threshold), so float64 gives the
    same answer: they must match exactly.
  * A DFL distance d = N / S with N = sum b e_b, S = sum e_b over 16 bins.
    Each e_b = exp(x_b - m) carries the rounding of x_b - m (relative error
    of e_b at most |x_b - m| u) and the exponential's own error (at most 2
    ulp, i.e. 4u relative; pinned against math.exp in the oracle tests).  A
    relative perturbation theta_b of each weight moves d by at most
    sum |b - d| w_b |theta_b| / S; with w_b = e^{-|x_b - m|} <= 1, S >= 1,
    |b - d| <= 15 and t e^{-t} <= 1/e this is at most 15 (16/e + 4) u.  The
    sums of 16 positive terms, the 16 products b e_b and the division add at
    most (15 + 16 + 1) u relative, i.e. 32 * 15 u absolute.  Hence
    |d32 - d| <= DFL_BOUND = 1.01 * (15 * (16 / e + 4) + 480) u ~ 3.8e-5 bin.
  * A box coordinate (c -+ d) * s: c is a cell centre (exact), the
    subtraction rounds once (u |c -+ d|), and the stride is a power of two
    (exact).  So |x32 - x| <= s (DFL_BOUND + u |c -+ d|) =: delta.
  * Mapping to source pixels, (x - left) * sx with sx = binary32(W / rw),
    then clipping (1-Lipschitz): at most sx delta plus 3u of the mapped
    magnitude (one subtraction, the rounding of sx, one product).
  * IoU of two binary32 boxes whose coordinates are within delta of the
    exact ones: the intersection's sides move by at most 2 delta and the
    areas by at most 2 delta (w + h) + 4 delta^2, so
    |IoU' - IoU| <= (dI + dU) / (U - dU) with dI <= 2 delta (iw + ih) +
    4 delta^2 and dU <= dA_a + dA_b + dI; evaluating IoU in binary32 adds
    at most 16u (areas 3u, intersection 3u, union 12u relative to U, the
    division u).  A suppression decision is called in-band when
    |IoU_exact - thr| is within that bound: there binary32 may decide
    either way, and the result's own decision is taken.  Outside the band
    the decision must be the exact one.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import detect as D

U = 2.0 ** -24
DFL_BOUND = 1.01 * (15 * (16 / math.e + 4) + 480) * U
F32 = np.float32


def exact_candidates(head, net_w, net_h, conf_thr):
    """Rank-ordered candidates from the float64 definitions: list of dicts
    with anchor, class, probability (binary32 input value), the exact
    network-input box (float64) and its per-coordinate error bound delta."""
    head = np.asarray(head, dtype=F32)
    nc = head.shape[0] - 4 * D.REG_MAX
    probs = head[4 * D.REG_MAX:].astype(np.float64)
    anc = D.anchors(net_w, net_h)
    thr = float(F32(conf_thr))
    out = []
    for a in range(head.shape[1]):
        col = probs[:, a]
        best_c, best_p = 0, -math.inf
        for c in range(nc):          # first maximum; NaN never wins
            if col[c] > best_p:
                best_c, best_p = c, col[c]
        if not best_p > thr:
            continue
        cx, cy, s = anc[a]
        d = [D.dfl_exact(head[side * D.REG_MAX:(side + 1) * D.REG_MAX, a].astype(np.float64))
             for side in range(4)]
        box = ((cx - d[0]) * s, (cy - d[1]) * s, (cx + d[2]) * s, (cy + d[3]) * s)
        mags = (abs(cx - d[0]), abs(cy - d[1]), abs(cx + d[2]), abs(cy + d[3]))
        delta = max(s * (DFL_BOUND + U * m) for m in mags)
        out.append({"anchor": a, "cls": best_c, "p": best_p, "box": box, "delta": delta})
    out.sort(key=lambda c: (-c["p"], c["anchor"]))
    return out


def iou_band(a, b, da, db):
    """Bound on |binary32 IoU - exact IoU| for exact boxes a, b whose
    binary32 coordinates lie within da, db of them."""
    d = max(da, db)
    wa, ha = a[2] - a[0], a[3] - a[1]
    wb, hb = b[2] - b[0], b[3] - b[1]
    iw = max(0.0, min(a[2], b[2]) - max(a[0], b[0]))
    ih = max(0.0, min(a[3], b[3]) - max(a[1], b[1]))
    inter = iw * ih
    union = wa * ha + wb * hb - inter
    di = 2 * d * (iw + ih) + 4 * d * d
    du = 2 * d * (wa + ha) + 2 * d * (wb + hb) + 8 * d * d + di
    if union - du <= 0:
        return math.inf
    return (di + du) / (union - du) * 1.01 + 16 * U * 1.01 + 1e-12


def mapped_exact(box, region, src_w, src_h):
    """Exact box in source pixels and the bound's mapping part."""
    left, top, rw, rh = region
    sx, sy = src_w / rw, src_h / rh
    x1 = min(max((box[0] - left) * sx, 0.0), src_w)
    y1 = min(max((box[1] - top) * sy, 0.0), src_h)
    x2 = min(max((box[2] - left) * sx, 0.0), src_w)
    y2 = min(max((box[3] - top) * sy, 0.0), src_h)
    return (x1, y1, x2, y2), max(sx, sy)


def check_against_definitions(result, head, src_w, src_h, net_w, net_h, region, conf, iou,
                              max_det, agnostic):
    """Check a detection result (boxes [n][4] in source pixels, scores,
    classes, candidate count; kept boxes in keep order) against greedy NMS
    run on the float64 definitions.  Returns the number of suppression
    decisions that fell inside the binary32 band (taken from the result);
    raises AssertionError on any other difference."""
    boxes, scores, classes, ncand = result
    boxes = np.asarray(boxes, dtype=np.float64).reshape(-1, 4)
    cands = exact_candidates(head, net_w, net_h, conf)
    assert ncand == len(cands), f"candidates: result {ncand}, definition {len(cands)}"
    thr = Fraction(float(F32(iou)))
    kept, in_band, j = [], 0, 0

    def matches(c, j):
        if j >= len(scores):
            return False
        if int(classes[j]) != c["cls"] or float(F32(scores[j])) != c["p"]:
            return False
        ex, sx = mapped_exact(c["box"], region, src_w, src_h)
        bound = sx * c["delta"] * 1.01 + 4 * U * (max(abs(v) for v in ex) + 1.0)
        return bool(np.all(np.abs(boxes[j] - np.array(ex)) <= bound))

    for c in cands:
        if len(kept) == max_det:
            break
        verdict = "keep"
        for k in kept:
            if not (agnostic or k["cls"] == c["cls"]):
                continue
            ie = D.iou_exact(k["box"], c["box"])
            band = iou_band(k["box"], c["box"], k["delta"], c["delta"])
            if abs(float(ie - thr)) > band:
                if ie > thr:
                    verdict = "suppress"
                    break
            else:
                verdict = "band" if verdict == "keep" else verdict
        if verdict == "band":
            in_band += 1
            verdict = "keep" if matches(c, j) else "suppress"
        if verdict == "keep":
            assert matches(c, j), (f"kept box {j}: definition keeps anchor {c['anchor']} "
                                   f"(class {c['cls']}, p {c['p']}), result differs")
            kept.append(c)
            j += 1
    assert j == len(scores), f"result keeps {len(scores)} boxes, definition {j}"
    return in_band
