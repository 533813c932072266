import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def read_golden(name):
    """Non-comment lines of a golden fixture, whitespace-split."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def ternarize_rounding_cases():
    """The hand-worked cases of ternarize_rounding.txt as dicts with the master
    weights W (fp32 [N,K]), the expected codes (int8 [N,K]) and the expected
    scale (a float)."""
    import numpy as np
    ex, cur = [], None
    for r in read_golden("ternarize_rounding.txt"):
        if r[0] == "example":
            cur = {"name": r[1], "set": [], "code": []}
            ex.append(cur)
        elif r[0] in ("N", "K"):
            cur[r[0]] = int(r[1])
        elif r[0] == "fill":
            cur["fill"] = float.fromhex(r[1])
        elif r[0] == "set":
            cur["set"].append((int(r[1]), int(r[2]), float.fromhex(r[3])))
        elif r[0] == "scale":
            cur["scale"] = float.fromhex(r[1])
        elif r[0] == "fill_code":
            cur["fill_code"] = int(r[1])
        elif r[0] == "code":
            cur["code"].append((int(r[1]), int(r[2]), int(r[3])))
    for e in ex:
        W = np.full((e["N"], e["K"]), e["fill"], np.float32)
        C = np.full((e["N"], e["K"]), e["fill_code"], np.int8)
        for n, k, v in e["set"]:
            W[n, k] = v
        for n, k, c in e["code"]:
            C[n, k] = c
        e["W"], e["codes"] = W, C
    return ex
