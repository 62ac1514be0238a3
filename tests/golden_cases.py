"""Loader for ``tests/golden/hand_derived.json``: hand-worked cases, padded
with zeros to the block length (zeros change neither absmax nor any code)."""
import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_derived.json")


def load():
    with open(PATH) as f:
        return json.load(f)


def pad(values, block, dtype=np.float32):
    a = np.zeros(block, dtype)
    a[:len(values)] = values
    return a


def bits_to_f32(h: str) -> np.float32:
    return np.uint32(int(h, 16)).view(np.float32)


PATH_E4M3 = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_derived_e4m3.json")


def load_e4m3():
    with open(PATH_E4M3) as f:
        return json.load(f)


def e4m3_x(case, block):
    """A case's input block (from "x" or "x_bits"), zero-padded."""
    if "x_bits" in case:
        vals = [bits_to_f32(h) for h in case["x_bits"]]
    else:
        vals = case["x"]
    return pad(np.asarray(vals, np.float32), block)


def e4m3_bytes(hexes):
    return [int(h, 16) for h in hexes]


def e4m3_scale(case):
    return bits_to_f32(case["scale_bits"]) if "scale_bits" in case else np.float32(case["scale"])


def e4m3_dequant_bits(case):
    if "dequant_bits" in case:
        return [int(h, 16) for h in case["dequant_bits"]]
    return list(np.asarray(case["dequant"], np.float32).view(np.uint32))
