"""Readers of the hand-derived fixtures under tests/golden/ (no arithmetic of
the method: the values are parsed as written)."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_unfused_cases():
    """Cases of combine_unfused_cases.txt: two-slot tokens with the bf16 bits
    of y, the float32 weights, and the expected bf16 output of the separately
    rounded and of the fused evaluation."""
    cases = []
    with open(os.path.join(GOLDEN, "combine_unfused_cases.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, y0, y1, w0, w1, sep, fused = line.split()
            w = np.array([int(w0, 16), int(w1, 16)], dtype=np.uint32).view(np.float32)
            cases.append({"name": name, "y": [int(y0, 16), int(y1, 16)], "w": w,
                          "unfused": int(sep, 16), "fused": int(fused, 16)})
    return cases
