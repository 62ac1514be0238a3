"""The oracle on the hand-derived E4M3 cases of
tests/golden/hand_derived_e4m3.json.  No GPU."""
import numpy as np

import golden_cases as gc


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_golden_e4m3_quantize(oracle_lib):
    g = gc.load_e4m3()
    B = g["block"]
    for case in g["quantize"]:
        x = gc.e4m3_x(case, B)
        codes, scales = oracle_lib.quantize_e4m3(x, B)
        assert _bits(scales[0]) == _bits(gc.e4m3_scale(case)), case["name"]
        want = gc.e4m3_bytes(case["codes"])
        assert list(codes[:len(want)]) == want, case["name"]
        assert not codes[len(want):].any()
        y = oracle_lib.dequantize_e4m3(codes, scales, B, "f32")
        assert list(_bits(y[:len(want)])) == gc.e4m3_dequant_bits(case), case["name"]


def test_golden_e4m3_reduce(oracle_lib):
    g = gc.load_e4m3()
    B = g["block"]
    for case in g["reduce"]:
        qs = [oracle_lib.quantize_e4m3(gc.pad(r, B), B) for r in case["ranks"]]
        for (c, _), want in zip(qs, case["rank_codes"]):
            assert list(c[:len(want)]) == gc.e4m3_bytes(want), case["name"]
        oc, os_ = oracle_lib.reduce_e4m3([q[0] for q in qs], [q[1] for q in qs], B)
        assert os_[0] == np.float32(case["scale"]), case["name"]
        assert list(oc[:len(case["codes"])]) == gc.e4m3_bytes(case["codes"]), case["name"]
        y = oracle_lib.dequantize_e4m3(oc, os_, B, "f32")
        assert np.array_equal(y[:len(case["dequant"])], np.float32(case["dequant"])), case["name"]


def test_golden_e4m3_ring_step(oracle_lib):
    g = gc.load_e4m3()
    B = g["block"]
    for case in g["ring_step"]:
        codes = gc.pad(gc.e4m3_bytes(case["codes_in"]), B, np.uint8)
        oc, os_ = oracle_lib.ring_step_e4m3(codes, np.float32([case["scale_in"]]), gc.pad(case["local"], B), B)
        assert os_[0] == np.float32(case["scale"]), case["name"]
        assert list(oc[:len(case["codes"])]) == gc.e4m3_bytes(case["codes"]), case["name"]
