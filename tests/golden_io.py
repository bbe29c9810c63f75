"""Reader for the hand-derived fixtures under tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.split()
    rows, cols = int(d["rows"][0]), int(d["cols"][0])
    x = np.array([float(t) for t in d["x"]], dtype=np.float32).reshape(rows, cols)
    # '-0' must keep its sign
    for i, t in enumerate(d["x"]):
        if t.strip() == "-0":
            x.reshape(-1)[i] = np.float32(-0.0)
    return {
        "x": x,
        "s_t_bits": int(d["s_t_bits"][0], 16),
        "scales": np.array([int(t, 16) for t in d["scales"]], dtype=np.uint8).reshape(rows, -1),
        "codes": np.array([int(t, 16) for t in d["codes"]], dtype=np.uint8).reshape(rows, -1),
    }


def names():
    return sorted(f for f in os.listdir(GOLDEN) if f.endswith(".txt") and f != "README.txt")
