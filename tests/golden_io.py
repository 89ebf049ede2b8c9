"""Read the worked-example fixture (values stored as exact rationals / 'ln(x)')."""
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _val(s: str) -> float:
    s = s.strip()
    if s == "-inf":
        return -math.inf
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _val(x)


def load_worked_example():
    with open(os.path.join(GOLDEN_DIR, "worked_example.json")) as f:
        raw = json.load(f)
    out = {}
    for key, ent in raw.items():
        if key in ("causal", "bottom_right"):
            out[key] = {k: _arr(v["value"]) for k, v in ent.items()}
        elif isinstance(ent, dict) and "value" in ent:
            v = ent["value"]
            out[key] = _arr(v) if isinstance(v, list) else _val(v)
    return out
