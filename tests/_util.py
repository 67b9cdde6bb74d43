"""Test helpers: the output tolerance metric and the golden-fixture reader."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerance on f32 outputs: per-element error relative to max(|r_n|, rms(r)).
REL_TOL = 1e-3


def rel_err(y, r):
    """max_n |y_n - r_n| / max(|r_n|, rms(r)): a per-element relative error
    whose denominator is floored at the RMS of the reference, because outputs
    that sit near zero make a pure ratio ill-posed."""
    y = np.asarray(y, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms)
    den[den == 0] = 1.0
    return float(np.max(np.abs(y - r) / den))


def read_golden(name):
    """key: value fixture; 'bytes:' may continue over following hex lines."""
    out, key = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            if ":" in line and not all(c in "0123456789abcdef" for c in line.strip()):
                key, val = line.split(":", 1)
                key = key.strip()
                out.setdefault(key, []).append(val.strip())
            else:
                out[key][-1] += line.strip()
    return out
