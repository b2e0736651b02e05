"""Reader for the small text fixtures in this folder (``key = numbers`` lines,
``#`` comments carry the citation and derivation)."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, vals = line.partition("=")
            out[key.strip()] = np.array([float(v) for v in vals.split()], dtype=np.float64)
    return out
