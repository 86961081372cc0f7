"""Loader for the page-value fixtures under tests/golden/ (plain text).

Format: '#' comment lines (each file starts with its citation), then
'name = values' lines; rows of a matrix are separated by ';'.
"""
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN_DIR, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            rows = [[float(t) for t in r.split()] for r in val.split(";")]
            arr = np.array(rows, dtype=np.float64)
            out[key] = arr if len(rows) > 1 else (arr[0] if arr.shape[1] > 1 else float(arr[0, 0]))
    return out
