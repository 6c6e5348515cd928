"""Readers for tests/golden/: the hand-worked fixtures (text) and the
oracle's stored direct solutions of the full-size workloads (``.npz``
written by ``golden/make_oracle_solutions.py``)."""
from __future__ import annotations

import hashlib
import os
from fractions import Fraction
from typing import Dict, Optional

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


def input_digest(wl) -> str:
    """SHA-256 over the bytes of a workload's L, Psi, g and B (in that order)."""
    h = hashlib.sha256()
    for a in (wl.L, wl.Psi, wl.g, wl.B):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def oracle_solutions_path(name: str) -> str:
    return os.path.join(GOLDEN, "oracle_%s.npz" % name)


def load_oracle_solutions(name: str) -> Optional[Dict[str, np.ndarray]]:
    """The stored oracle solutions of workload ``name`` (None if absent)."""
    path = oracle_solutions_path(name)
    if not os.path.exists(path):
        return None
    with np.load(path, allow_pickle=False) as d:
        return {k: d[k] for k in d.files}
