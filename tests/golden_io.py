"""Reader for the small text fixtures under tests/golden/ (``key: values``
lines, ``;`` separating matrix rows, ``#`` comments)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            rows = [r.split() for r in v.split(";")]
            vals = [[float(t) for t in r] for r in rows]
            if len(vals) == 1 and len(vals[0]) == 1:
                out[k.strip()] = vals[0][0]
            else:
                out[k.strip()] = np.array(vals[0] if len(vals) == 1 else vals, dtype=np.float64)
    return out
