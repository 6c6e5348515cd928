"""Reader for the hand-worked fixtures under tests/golden/."""
from __future__ import annotations

import os
from fractions import Fraction
from typing import Dict

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok: str) -> Fraction:
    return Fraction(tok)


def _parse_value(text: str):
    rows = [r.split() for r in text.split(";")]
    vals = [[_num(t) for t in r] for r in rows]
    if len(vals) == 1:
        return vals[0] if len(vals[0]) > 1 else vals[0][0]
    return vals


def load(name: str) -> Dict[str, object]:
    out: Dict[str, object] = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = [s.strip() for s in line.split("=", 1)]
            out[key] = _parse_value(val)
    return out


def as_float(v) -> np.ndarray:
    return np.array(v, dtype=object).astype(np.float64)
