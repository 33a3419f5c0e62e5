"""Loads the hand-derived fixtures under tests/golden/ (no arithmetic of the
method here: fractions and the value ln 3 are turned into numbers)."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LN3 = math.log(3.0)


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def logits_f32(fx: dict) -> np.ndarray:
    """The fixture's logits as float32 ("ln3" is the float32 rounding of ln 3)."""
    return np.array([[np.float32(LN3) if v == "ln3" else np.float32(v) for v in row]
                     for row in fx["logits"]], dtype=np.float32)


def fraction(s: str) -> float:
    return float(Fraction(s))


def closed_form(expr: str) -> float:
    """A closed-form value written with numbers, + - * / ( ) and ln3."""
    allowed = set("0123456789.+-*/() ")
    body = expr.replace("ln3", "")
    if not set(body) <= allowed:
        raise ValueError(f"unexpected token in {expr!r}")
    return float(eval(expr, {"__builtins__": {}}, {"ln3": LN3}))  # noqa: S307 (checked above)
