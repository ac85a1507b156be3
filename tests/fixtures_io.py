"""Loads the hand-worked fixtures of tests/golden into round inputs."""
import glob
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fixture_names():
    return sorted(os.path.basename(p)[:-5] for p in glob.glob(os.path.join(GOLDEN, "*.json")))


def load(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        g = json.load(f)
    w = {k: np.asarray(v, dtype=np.float32) for k, v in g["weights"].items()}
    inputs = {"weights": w, "H": np.asarray(g["H"], np.float32),
              "root": np.asarray(g["root"], np.int32), "wtype": "f32"}
    env = {"ln2": math.log(2.0), "log": math.log}
    exp = dict(g["expect"])
    exp["score"] = [float(eval(sx, {"__builtins__": {}}, env)) for sx in exp["score"]]
    return g, inputs, exp
