"""Loader for the hand-worked d=4 golden case (tests/golden/toy_d4.json)."""
import json
import math
import os

import numpy as np

from oracle.numerics import round_to_bf16

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "toy_d4.json")


def _val(x):
    if isinstance(x, str):
        e = math.e
        return float(eval(x.replace("2e", "2*e"), {"__builtins__": {}}, {"e": e}))
    return float(x)


def load():
    with open(PATH) as f:
        g = json.load(f)
    for c in g["cases"]:
        if c["out"] is not None:
            c["out"] = np.array([[_val(v) for v in row] for row in c["out"]], dtype=np.float64)
    return g


def padded(g, d=128, r=16):
    """Embed the toy in d / r by zero padding: extra basis rows are unit vectors on
    coordinates the toy never uses, so every score and logit is unchanged."""
    q = np.zeros((len(g["q_heads"]), d))
    q[:, :4] = g["q_heads"]
    K = np.zeros((len(g["K"]), d))
    K[:, :4] = g["K"]
    V = np.zeros((len(g["V"]), d))
    V[:, :4] = g["V"]
    M = np.zeros((r, d), dtype=np.float32)
    M[:2, :4] = g["M"]
    for i in range(2, r):
        M[i, 4 + i] = 1.0
    return round_to_bf16(q), round_to_bf16(K), round_to_bf16(V), M
