"""The seeded input generator: deterministic, the recipe's shapes, types and
statistics.  No GPU."""
import json
import os

import numpy as np
import pytest

from block_wise_int8_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fingerprints_stable():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mk", os.path.join(HERE, "golden", "make_synth_hashes.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(HERE, "golden", "synth_sha256.json")) as f:
        stored = json.load(f)
    assert mk.fingerprints() == stored


@pytest.mark.parametrize("key", sorted(synth.WORKLOADS))
def test_recipe_shapes(key):
    w = synth.WORKLOADS[key]
    small = w.resized(n=4096) if len(w.shape) == 1 else w.resized(rows=4)
    rs = synth.ranks(small)
    assert len(rs) == w.nranks
    for r in rs:
        assert r.shape == (small.n,)
        assert r.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
    assert small.n % w.block == 0


def _f(x):
    return (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x


def test_recipe_statistics():
    r = _f(synth.ranks(synth.WORKLOADS["tiny"])[0])
    assert abs(r.mean()) < 0.1 and abs(r.std() - 1) < 0.1
    w = synth.WORKLOADS["outliers"].resized(n=1 << 20)
    x = _f(synth.ranks(w.resized(nranks=1))[0])
    assert (np.abs(x) > 8).sum() > 0.8 * (w.n // 1000)          # most outliers exceed 8 sigma
    w = synth.WORKLOADS["ring"].resized(rows=64)
    x = _f(synth.ranks(w.resized(nranks=1))[0])
    assert np.abs(np.median(np.abs(x)) - 0.5 * np.log(2)) < 0.02   # Laplace(0, b) median |x| = b ln 2
    w = synth.WORKLOADS["smallblock"].resized(n=1 << 16)
    x = synth.ranks(w.resized(nranks=1))[0].reshape(-1, 64)
    spread = np.log(np.abs(x).max(axis=1))
    assert spread.std() > 1.5                                    # per-block lognormal(0, 2) magnitudes


def test_bf16_conversion_is_rne():
    f = np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)])
    assert list(synth.f32_to_bf16_bits(f)) == [0x3F80, 0x3F82, 0xBF80]
