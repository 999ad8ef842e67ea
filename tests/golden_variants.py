"""Loaders for the hand-worked gated-logit and block-sparse cases
(tests/golden/gated_toy.json, tests/golden/block_toy.json). Values written as
expressions use e, ln2 and ln3 only."""
import json
import math
import os

import numpy as np

from oracle.numerics import round_to_bf16

DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_NAMES = {"e": math.e, "ln2": math.log(2.0), "ln3": math.log(3.0)}


def value(x) -> float:
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, dict(_NAMES)))
    return float(x)


def matrix(rows) -> np.ndarray:
    return np.array([[value(v) for v in row] for row in rows], dtype=np.float64)


def load(name: str) -> dict:
    with open(os.path.join(DIR, name + ".json")) as f:
        return json.load(f)


def padded_bits(rows, d=128) -> np.ndarray:
    """bf16 bits of the toy rows, zero padded to d (the extra dimensions change no dot product)."""
    a = np.zeros((len(rows), d))
    a[:, :len(rows[0])] = rows
    return round_to_bf16(a)
