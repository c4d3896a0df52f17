"""Writes tests/golden/tiny_t1_seed0.json: the NumPy oracle's outputs on the
seeded tiny workload (one token, H=256, 8 experts top-2, I=Is=128, fp32 block
scales), plus a SHA-256 of every input tensor.  Calls only synth/ and oracle/.

The pages print no worked example of their own, so this file is a regression
record of the oracle, not an independent pin: the pins live in
tests/test_oracle_pins.py.

Run from the repository root:  python tests/golden/make_golden.py
"""

import dataclasses
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from synth import WORKLOADS, make_layer  # noqa: E402

NAME = "tiny_t1"


def input_digests(inp):
    out = {}
    for f in dataclasses.fields(inp):
        v = getattr(inp, f.name)
        if isinstance(v, np.ndarray):
            out[f.name] = hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
    return out


def main():
    inp = make_layer(WORKLOADS[NAME], seed=0)
    r = oracle.moe_layer(inp)
    rec = {
        "workload": NAME,
        "seed": 0,
        "inputs_sha256": input_digests(inp),
        "ids": r["ids"].tolist(),
        "weights": r["weights"].tolist(),
        "gaps": r["gaps"].tolist(),
        "h": r["h"].tolist(),
        "out": r["out"].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), NAME + "_seed0.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
