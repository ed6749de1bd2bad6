"""CPU oracle for the fixed-shape frame pipeline -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct restatement of what the pipeline computes,
written from the WarpStream TRT article (fused-preprocess passage and its
dataflow figure; the Top-K passage) and the yolo.cu README (letterboxed
input; DFL decode and greedy NMS), in float64 with exact rational sampling
coordinates.  Detection decisions are taken in binary32 with a fixed
operation order (oracle/detect.py says why).

Only the test-suite, the package's smoke entry point and the benchmark's CPU
baseline leg may import this package.  The HIP library never does, and this
package imports nothing from it: the two share no code.

Parity pins (what ties this oracle to the pages and the mathematics, not to
itself) live in tests/test_oracle_*.py.  Every function here is pinned; none
is "parity unpinned" except the two letterbox readings listed in
oracle/preprocess.py (odd pad split and non-integer scaled size), which no
workload exercises.
"""
from .preprocess import axis_taps, letterbox_region, preprocess, preprocess_batch, pad_value
from .topk import topk, topk_keys_order
from . import detect

__all__ = ["axis_taps", "letterbox_region", "preprocess", "preprocess_batch", "pad_value",
           "topk", "topk_keys_order", "detect"]
