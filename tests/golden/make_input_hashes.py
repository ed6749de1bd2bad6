"""Writes input_sha256.json: SHA-256 of every seeded workload input.

Calls only the seeded input generators (no pipeline arithmetic), so the stored
hashes pin input determinism: the same seeds must yield the same bytes on any
host that runs the tests or the benchmark.
Run from the repository root:  python tests/golden/make_input_hashes.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from post_processing_amd import workloads as wl  # noqa: E402


def hashes():
    out = {}
    for name, fn in wl.ALL_CONFIGS.items():
        w = fn()
        out[name] = {"frames": wl.sha256(w.frames), "scores": wl.sha256(w.scores)}
    for lane in range(8):
        w = wl.c5_lane(lane)
        out[f"c5_lane{lane}"] = {"frames": wl.sha256(w.frames), "scores": wl.sha256(w.scores)}
    w = wl.c5_throughput(64)
    out["c5t"] = {"frames": wl.sha256(w.frames)}
    w = wl.c3d()
    out["c3d"] = {"frames": wl.sha256(w.frames), "head": wl.sha256(w.head)}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_sha256.json")
    with open(path, "w") as f:
        json.dump(hashes(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)
