"""Write datagen_sha256.json: SHA-256 of the seeded input bytes of each
workload (Tiny in full; the first heads of the larger ones), so that any
change to the input recipe shows up in the CPU tests.

Usage (from the repository root): python tests/golden/make_datagen_hashes.py
It calls only the input generator; no step of the method runs here.
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import datagen  # noqa: E402

SLICES = [("tiny", None), ("480p", 2), ("720p", 2), ("hc", 3), ("long", 1)]


def hashes():
    out = {}
    for name, heads in SLICES:
        w = datagen.WORKLOADS[name]
        if heads is not None:
            w = w.with_heads(heads)
        data = datagen.generate(w)
        key = name if heads is None else f"{name}/heads0-{heads - 1}"
        out[key] = {t: hashlib.sha256(data[t].tobytes()).hexdigest() for t in ("q", "k", "v", "wq", "wk")}
    return out


if __name__ == "__main__":
    doc = {"source": "seeded input generator (datagen), recipe in its module docstring; "
                     "numpy PCG64 streams and float64 math on this image",
           "hashes": hashes()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "datagen_sha256.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
