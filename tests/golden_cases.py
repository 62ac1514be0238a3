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
