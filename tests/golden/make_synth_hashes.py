"""Writes synth_sha256.json: SHA-256 fingerprints of the seeded generator's
rank buffers (small instances of every recipe), so that a change of draw
order, seed or conversion shows up.  Calls only the generator."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from block_wise_int8_amd import synth  # noqa: E402

SMALL = {
    "tiny": {},
    "outliers": {"n": 1 << 16},
    "prefill": {"rows": 8},
    "ring": {"rows": 8},
    "smallblock": {"n": 1 << 14},
}


def fingerprints():
    out = {}
    for key, kw in SMALL.items():
        w = synth.WORKLOADS[key].resized(**kw) if kw else synth.WORKLOADS[key]
        out[key] = {"resize": kw, "sha256": [synth.sha256(r) for r in synth.ranks(w)]}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_sha256.json")
    with open(path, "w") as f:
        json.dump(fingerprints(), f, indent=1)
    print("wrote", path)
