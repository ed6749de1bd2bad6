"""Seeded synthetic inputs for the frame pipeline (frames and score vectors).

This module draws random numbers and nothing else: it holds none of the
pipeline's arithmetic (no sampling, normalisation, letterbox placement,
decode or selection), so both the CPU oracle's tests and the HIP path can
take their inputs from it.  Where planted detection objects need a window
of the network canvas, the window is a constant given by the caller.

Workload shapes follow the WarpStream TRT article (batch-1 interleaved RGB8
producer frames, fixed-size FP32 classifier logits, Top-K with K <= 32) and the
yolo.cu README (640x640 letterbox input, 8400 anchors x 80 classes):

  C1  64x48 RGB8 -> 32x32 resize, K=5 over 1000 logits with 10 planted ties
  C2  1920x1080 RGB8 (uniform + gradient) -> 224x224, K=5 over 1000 logits
  C3  1280x720 RGB8 -> 640x640 letterbox (pad 114, /255 only),
      K=32 over 8400x80 sigmoid scores
  C4  3840x2160 RGB8 -> 384x384, K=32 over 21843 logits with 1% exact copies
  C5L 8 lanes of C2-shaped frames read from mapped host memory, K=10
  C5T 64 independent 1280x720 frames -> 224x224 (preprocess only)
  C3D C3's frame geometry plus a YOLO-style detection head (4x16 DFL logits
      + 80 class probabilities per anchor, 8400 anchors) with planted objects

Every generator uses numpy.random.default_rng(seed) (PCG64) and draws in the
order frame, scores, duplicate positions.  Widths are given first ("W x H"),
so frame arrays have shape (H, W, 3).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

IMAGENET_MEAN = (0.485, 0.456, 0.406)
IMAGENET_STD = (0.229, 0.224, 0.225)

RESIZE = 0
LETTERBOX = 1


@dataclass
class Workload:
    """One pipeline configuration plus its seeded inputs."""

    name: str
    src_w: int
    src_h: int
    dst_w: int
    dst_h: int
    mode: int                     # RESIZE or LETTERBOX
    mean: tuple                   # unit range, per RGB channel
    std: tuple
    pad: float                    # letterbox pad value in byte units
    k: int                        # 0 = no Top-K stage
    frames: np.ndarray            # uint8 [B][H][W][3]
    scores: np.ndarray | None     # float32 [N] or None
    host_input: bool = False      # frame read from mapped pinned host memory
    meta: dict = field(default_factory=dict)
    head: np.ndarray | None = None  # float32 [64 + nc][A] detection head, or None
    det: dict = field(default_factory=dict)   # nc, conf, iou, max_det, agnostic, planted

    @property
    def batch(self) -> int:
        return int(self.frames.shape[0])

    @property
    def num_scores(self) -> int:
        return 0 if self.scores is None else int(self.scores.shape[0])


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def uniform_frame(rng: np.random.Generator, w: int, h: int) -> np.ndarray:
    return rng.integers(0, 256, size=(h, w, 3), dtype=np.uint8)


def gradient_frame(rng: np.random.Generator, w: int, h: int) -> np.ndarray:
    """Uniform random bytes averaged with a smooth per-channel ramp.

    Ramp: R rises along x, G along y, B along the diagonal; the blend is
    (u + g) >> 1 in 16-bit integers.
    """
    u = uniform_frame(rng, w, h).astype(np.uint16)
    xs = np.arange(w, dtype=np.int64)
    ys = np.arange(h, dtype=np.int64)
    g = np.empty((h, w, 3), dtype=np.uint16)
    g[..., 0] = ((255 * xs) // max(w - 1, 1))[None, :]
    g[..., 1] = ((255 * ys) // max(h - 1, 1))[:, None]
    g[..., 2] = (255 * (xs[None, :] + ys[:, None])) // max(w + h - 2, 1)
    return ((u + g) >> 1).astype(np.uint8)


def plant_duplicates(rng: np.random.Generator, s: np.ndarray, sources: np.ndarray) -> np.ndarray:
    """Copy s[sources[j]] onto distinct random positions that are not sources."""
    s = s.copy()
    mask = np.ones(s.shape[0], dtype=bool)
    mask[sources] = False
    free = np.flatnonzero(mask)
    dst = rng.choice(free, size=sources.shape[0], replace=False)
    s[dst] = s[sources]
    return s


def normal_logits(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.standard_normal(n).astype(np.float32)


def c1(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    frame = uniform_frame(rng, 64, 48)
    s = normal_logits(rng, 1000)
    top10 = np.argsort(-s.astype(np.float64), kind="stable")[:10]
    s = plant_duplicates(rng, s, top10)
    return Workload("c1_64x48_to_32", 64, 48, 32, 32, RESIZE, IMAGENET_MEAN, IMAGENET_STD,
                    114.0, 5, frame[None], s)


def c2(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    frame = gradient_frame(rng, 1920, 1080)
    s = normal_logits(rng, 1000)
    return Workload("c2_1920x1080_to_224", 1920, 1080, 224, 224, RESIZE, IMAGENET_MEAN,
                    IMAGENET_STD, 114.0, 5, frame[None], s)


def c3(seed: int = 2) -> Workload:
    rng = np.random.default_rng(seed)
    frame = uniform_frame(rng, 1280, 720)
    x = rng.normal(-4.0, 2.0, 8400 * 80)
    s = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
    return Workload("c3_1280x720_letterbox_640", 1280, 720, 640, 640, LETTERBOX,
                    (0.0, 0.0, 0.0), (1.0, 1.0, 1.0), 114.0, 32, frame[None], s)


def c4(seed: int = 3) -> Workload:
    rng = np.random.default_rng(seed)
    frame = uniform_frame(rng, 3840, 2160)
    n = 21843
    s = normal_logits(rng, n)
    ndup = int(round(0.01 * n))
    order = np.argsort(-s.astype(np.float64), kind="stable")
    top = order[:32]
    rest = rng.choice(order[32:], size=ndup - 32, replace=False)
    s = plant_duplicates(rng, s, np.concatenate([top, rest]))
    return Workload("c4_3840x2160_to_384", 3840, 2160, 384, 384, RESIZE, IMAGENET_MEAN,
                    IMAGENET_STD, 114.0, 32, frame[None], s)


def c5_lane(lane: int) -> Workload:
    rng = np.random.default_rng(40 + lane)
    frame = gradient_frame(rng, 1920, 1080)
    s = normal_logits(rng, 1000)
    return Workload(f"c5_lane{lane}_1920x1080_to_224", 1920, 1080, 224, 224, RESIZE,
                    IMAGENET_MEAN, IMAGENET_STD, 114.0, 10, frame[None], s, host_input=True)


def c5_throughput(frames: int = 64) -> Workload:
    batch = np.empty((frames, 720, 1280, 3), dtype=np.uint8)
    for i in range(frames):
        batch[i] = uniform_frame(np.random.default_rng(1000 + i), 1280, 720)
    return Workload(f"c5t_{frames}x1280x720_to_224", 1280, 720, 224, 224, RESIZE,
                    IMAGENET_MEAN, IMAGENET_STD, 114.0, 0, batch, None)


def random_small(seed: int, letterbox: bool = False, max_side: int = 67) -> Workload:
    """Small random shapes (source and destination sides 1..max_side) for edge cases."""
    rng = np.random.default_rng(10_000 + seed)
    sw, sh, dw, dh = (int(v) for v in rng.integers(1, max_side + 1, size=4))
    batch = int(rng.integers(1, 4))
    frames = rng.integers(0, 256, size=(batch, sh, sw, 3), dtype=np.uint8)
    mean = tuple(float(v) for v in rng.uniform(0.0, 1.0, 3))
    std = tuple(float(v) for v in rng.uniform(0.1, 1.0, 3))
    pad = float(rng.integers(0, 256))
    return Workload(f"small{seed}_{sw}x{sh}_to_{dw}x{dh}{'_lb' if letterbox else ''}",
                    sw, sh, dw, dh, LETTERBOX if letterbox else RESIZE, mean, std, pad, 0,
                    frames, None)


def scores_with_specials(seed: int, n: int, tie_frac: float = 0.1, nan_frac: float = 0.0,
                         specials: bool = True) -> np.ndarray:
    """N(0,1) scores with planted exact ties, NaNs, +-0, +-inf and subnormals."""
    rng = np.random.default_rng(20_000 + seed)
    s = rng.standard_normal(n).astype(np.float32)
    if n == 0:
        return s
    nt = int(n * tie_frac)
    if nt:
        src = rng.integers(0, n, size=nt)
        dst = rng.integers(0, n, size=nt)
        s[dst] = s[src]
    nn = int(n * nan_frac)
    if nn:
        s[rng.integers(0, n, size=nn)] = np.nan
    if specials and n >= 8:
        pos = rng.choice(n, size=8, replace=False)
        vals = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1e-40, np.nan],
                        dtype=np.float32)
        s[pos] = vals
    return s


HEAD_BINS = 16            # DFL bins per box side
HEAD_STRIDES = (8, 16, 32)


def head_anchor_grid(net_w: int, net_h: int):
    """Anchor cell centres (cx, cy) in cells and strides, in head order:
    stride-8 grid, then 16, then 32, row-major within a grid."""
    cx, cy, st = [], [], []
    for s in HEAD_STRIDES:
        gy, gx = np.meshgrid(np.arange(net_h // s), np.arange(net_w // s), indexing="ij")
        cx.append(gx.ravel() + 0.5)
        cy.append(gy.ravel() + 0.5)
        st.append(np.full(gx.size, s, dtype=np.float64))
    return np.concatenate(cx), np.concatenate(cy), np.concatenate(st)


def detection_head(rng: np.random.Generator, net_w: int, net_h: int, nc: int, region,
                   objects: int, bg_mean: float = -7.0, bg_std: float = 1.5):
    """A synthetic head: background anchors with low class probabilities
    (sigmoid of N(bg_mean, bg_std)) and N(0, 1.5) box logits; each planted
    object lights up the anchors whose centre lies in the middle half of its
    box, on the grids where its larger side spans 3..20 cells, with a
    probability sigmoid(N(2, 1)) for its class and box logits peaked (a
    Gaussian bump of width 0.7 bins plus N(0, 0.2) noise) at the distances
    to the object's edges jittered by N(0, 0.15) cells.  Objects are boxes
    inside `region` = (left, top, w, h) with sides 12..45% of the region.
    Returns (head float32 [64 + nc][A], planted [(class, x1, y1, x2, y2)])."""
    cx, cy, st = head_anchor_grid(net_w, net_h)
    A = cx.size
    head = np.empty((4 * HEAD_BINS + nc, A), dtype=np.float32)
    head[:4 * HEAD_BINS] = rng.normal(0.0, 1.5, (4 * HEAD_BINS, A))
    head[4 * HEAD_BINS:] = 1.0 / (1.0 + np.exp(-rng.normal(bg_mean, bg_std, (nc, A))))
    left, top, rw, rh = region
    bins = np.arange(HEAD_BINS, dtype=np.float64)[:, None]
    planted = []
    for _ in range(objects):
        cls = int(rng.integers(0, nc))
        w = rw * rng.uniform(0.12, 0.45)
        h = rh * rng.uniform(0.12, 0.45)
        x1 = left + rng.uniform(0, rw - w)
        y1 = top + rng.uniform(0, rh - h)
        x2, y2 = x1 + w, y1 + h
        planted.append((cls, x1, y1, x2, y2))
        span = max(w, h) / st
        px, py = cx * st, cy * st
        hit = ((span >= 3) & (span <= 20) &
               (np.abs(px - (x1 + x2) / 2) <= w / 4) & (np.abs(py - (y1 + y2) / 2) <= h / 4))
        idx = np.flatnonzero(hit)
        if idx.size == 0:
            continue
        p = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, idx.size)))
        head[4 * HEAD_BINS + cls, idx] = p
        dist = np.stack([cx[idx] - x1 / st[idx], cy[idx] - y1 / st[idx],
                         x2 / st[idx] - cx[idx], y2 / st[idx] - cy[idx]])
        dist = np.clip(dist + rng.normal(0.0, 0.15, dist.shape), 0.0, HEAD_BINS - 1)
        for side in range(4):
            bump = -((bins - dist[side][None, :]) ** 2) / (2 * 0.7 ** 2)
            head[side * HEAD_BINS:(side + 1) * HEAD_BINS, idx] = (
                bump + rng.normal(0.0, 0.2, bump.shape))
    return head, planted


def c3d(seed: int = 5, objects: int = 24) -> Workload:
    """C3's geometry with a detection head: 1280x720 -> 640x640 letterbox,
    8400 anchors x 80 classes, conf > 0.25, IoU > 0.45, at most 300 boxes.
    The Top-K stage ranks the head's class block (the same 8400x80 scores)."""
    rng = np.random.default_rng(seed)
    frame = uniform_frame(rng, 1280, 720)
    # Objects are planted in canvas rows 140..500, a fixed window (the band a
    # 16:9 frame covers on a square canvas) given here as constants.
    head, planted = detection_head(rng, 640, 640, 80, (0, 140, 640, 360), objects)
    return Workload("c3d_1280x720_letterbox_640_detect", 1280, 720, 640, 640, LETTERBOX,
                    (0.0, 0.0, 0.0), (1.0, 1.0, 1.0), 114.0, 32, frame[None],
                    head[4 * HEAD_BINS:].ravel().copy(), head=head,
                    det=dict(nc=80, conf=0.25, iou=0.45, max_det=300, agnostic=False,
                             planted=planted))


def detect_small(seed: int) -> Workload:
    """Small random detection cases: network sides 32..256 (multiples of 32),
    1..120 classes, 0..12 objects, random thresholds, letterbox or resize,
    sometimes class-agnostic, sometimes a small max_det."""
    rng = np.random.default_rng(30_000 + seed)
    nw, nh = (int(v) * 32 for v in rng.integers(1, 9, size=2))
    sw, sh = (int(v) for v in rng.integers(8, 400, size=2))
    letterbox = bool(rng.integers(0, 2))
    nc = int(rng.integers(1, 121))
    # Objects are planted anywhere on the network canvas (in letterbox mode
    # some fall on the pad bands, so their boxes are clipped to the frame
    # when mapped back).
    head, planted = detection_head(rng, nw, nh, nc, (0, 0, nw, nh), int(rng.integers(0, 13)),
                                   bg_mean=float(rng.uniform(-7.0, -1.0)))
    frames = rng.integers(0, 256, size=(1, sh, sw, 3), dtype=np.uint8)
    det = dict(nc=nc, conf=float(np.float32(rng.uniform(0.05, 0.6))),
               iou=float(np.float32(rng.uniform(0.2, 0.9))),
               max_det=int(rng.choice([1, 3, 10, 300])), agnostic=bool(rng.integers(0, 2)),
               planted=planted)
    return Workload(f"detect_small{seed}_{sw}x{sh}_to_{nw}x{nh}", sw, sh, nw, nh,
                    LETTERBOX if letterbox else RESIZE, (0.0, 0.0, 0.0), (1.0, 1.0, 1.0),
                    114.0, 0, frames, None, head=head, det=det)


def uniform_head(seed: int, nw: int, nh: int, nc: int, conf: float, iou: float, max_det: int,
                 agnostic: bool = False, box_scale: float = 1.5) -> Workload:
    """A head whose class probabilities are uniform in [0, 1): about
    1 - conf**nc of the anchors become candidates (each anchor's best class
    is the largest of nc uniforms), with box logits N(0, box_scale).  Small
    box_scale flattens every side's DFL softmax, so all boxes are about 15
    cells wide and overlap their neighbours heavily."""
    rng = np.random.default_rng(50_000 + seed)
    A = head_anchor_grid(nw, nh)[0].size
    head = np.empty((4 * HEAD_BINS + nc, A), np.float32)
    head[:4 * HEAD_BINS] = rng.normal(0.0, box_scale, (4 * HEAD_BINS, A))
    head[4 * HEAD_BINS:] = rng.uniform(0.0, 1.0, (nc, A))
    frames = rng.integers(0, 256, size=(1, nh, nw, 3), dtype=np.uint8)
    return Workload(f"uniform_head{seed}", nw, nh, nw, nh, RESIZE, (0.0, 0.0, 0.0),
                    (1.0, 1.0, 1.0), 114.0, 0, frames, None, head=head,
                    det=dict(nc=nc, conf=conf, iou=iou, max_det=max_det, agnostic=agnostic))


def dense_detect(agnostic: bool = True) -> Workload:
    """The suppression stress case: a 1024x512 network (10,752 anchors), 80
    uniform classes with conf 0.75 (every anchor is a candidate), IoU > 0.3,
    up to 1,024 boxes, heavily overlapping boxes; by default boxes of any
    class suppress each other, so all candidates form one run."""
    w = uniform_head(2, 1024, 512, 80, 0.75, 0.3, 1024, agnostic=agnostic, box_scale=0.3)
    w.name = "dense_detect_1024x512_10752_anchors_" + ("any_class" if agnostic else "by_class")
    return w


ALL_CONFIGS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4}
