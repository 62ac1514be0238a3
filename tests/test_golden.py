"""The oracle on the hand-derived cases of tests/golden/hand_derived.json.
No GPU."""
import numpy as np

import golden_cases as gc
from block_wise_int8_amd import synth


def _f32bits(v):
    return np.float32(v).view(np.uint32)


def test_golden_quantize(oracle_lib):
    g = gc.load()
    B = g["block"]
    for case in g["quantize"]:
        x = gc.pad(case["x"], B)
        for xin in (x, synth.f32_to_bf16_bits(x)):
            codes, scales = oracle_lib.quantize(xin, B)
            want_s = gc.bits_to_f32(case["scale_bits"]) if "scale_bits" in case else np.float32(case["scale"])
            assert _f32bits(scales[0]) == _f32bits(want_s), case["name"]
            k = len(case["codes"])
            assert list(codes[:k]) == case["codes"], case["name"]
            assert not codes[k:].any()
            y = oracle_lib.dequantize(codes, scales, B, "f32")
            if "dequant" in case:
                assert np.array_equal(y[:k], np.float32(case["dequant"])), case["name"]
            for i, h in enumerate(case.get("dequant_bits", [])):
                if h is not None:
                    assert _f32bits(y[i]) == int(h, 16), (case["name"], i)


def test_golden_reduce(oracle_lib):
    g = gc.load()
    B = g["block"]
    for case in g["reduce"]:
        qs = [oracle_lib.quantize(gc.pad(r, B), B) for r in case["ranks"]]
        for (c, s), want_s in zip(qs, case["scales_in"]):
            assert s[0] == np.float32(want_s), case["name"]
        for (c, _), want_c in zip(qs, case.get("codes_in", [])):
            assert list(c[:len(want_c)]) == want_c, case["name"]
        oc, os_ = oracle_lib.reduce([q[0] for q in qs], [q[1] for q in qs], B)
        assert os_[0] == np.float32(case["scale"]), case["name"]
        assert list(oc[:len(case["codes"])]) == case["codes"], case["name"]
        y = oracle_lib.dequantize(oc, os_, B, "f32")
        assert np.array_equal(y[:len(case["dequant"])], np.float32(case["dequant"])), case["name"]


def test_golden_ring_step(oracle_lib):
    g = gc.load()
    B = g["block"]
    for case in g["ring_step"]:
        codes = gc.pad(case["codes_in"], B, np.int8)
        scales = np.float32([case["scale_in"]])
        local = synth.f32_to_bf16_bits(gc.pad(case["local"], B))
        oc, os_ = oracle_lib.ring_step(codes, scales, local, B)
        assert os_[0] == np.float32(case["scale"]), case["name"]
        assert list(oc[:len(case["codes"])]) == case["codes"], case["name"]
        y = oracle_lib.dequantize(oc, os_, B, "bf16")
        assert np.array_equal(y[:4], synth.f32_to_bf16_bits(np.float32(case["dequant"]))), case["name"]


def test_golden_negative_zero_dequantizes_to_plus_zero(oracle_lib):
    x = gc.pad([254, -0.0], 64)
    codes, scales = oracle_lib.quantize(x, 64)
    y = oracle_lib.dequantize(codes, scales, 64, "f32")
    assert _f32bits(y[1]) == 0
