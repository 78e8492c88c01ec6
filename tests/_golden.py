"""Load the hand-worked fixtures under tests/golden/ (values typed by hand)."""
import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LN3 = math.log(3.0)


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def num(x):
    """A fixture entry: a number, 'ln3', '2ln3' or a fraction string like '14/3'."""
    if isinstance(x, (int, float)):
        return float(x)
    if x == "ln3":
        return LN3
    if x == "2ln3":
        return 2.0 * LN3
    return float(Fraction(x))


def arr(nested, dtype=np.float64):
    if isinstance(nested, list):
        return np.array([arr(e, dtype) for e in nested], dtype=dtype)
    return num(nested)
