"""Reader for the small text fixtures under tests/golden/ (``key = row ; row`` lines)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            try:
                rows = [[float(v) for v in r.split()] for r in val.split(";")]
            except ValueError:
                out[key] = val
                continue
            arr = np.array(rows, dtype=np.float64)
            out[key] = arr[0, 0] if arr.size == 1 else (arr[0] if arr.shape[0] == 1 else arr)
    return out
