"""Helpers shared by the tests (no method arithmetic)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def golden_kv(name):
    out = {}
    for line in golden_lines(name):
        k, v = (s.strip() for s in line.split("=", 1))
        out[k] = float(v)
    return out


def max_rel_err(got, ref):
    """Max over output rows (the last axis is the row) of
    max|got - ref| / max|ref|: the tolerance metric of every parity test."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    num = np.abs(g2 - r2).max(axis=1)
    den = np.abs(r2).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    if not np.all(np.isfinite(g2)):
        return float("inf")
    return float((num / den).max()) if num.size else 0.0
