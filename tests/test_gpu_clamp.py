"""Blocks whose scale is subnormal, where the clamp of the rounded quotient
to [-Q, Q] binds (int8 Q = 127, E4M3 Q = 448, 4-bit Q = 7): s = fl(m / Q) can
lie well below m / Q there (m = 190 * 2^-149 gives s = 2^-149 and a quotient
of 190 for int8), so these blocks take the kernels' IEEE-division path with
its clamp.  Quantize, reduce, the one-kernel step and the ring step against
the oracle, bit for bit, with fp32 data that are exact multiples of 2^-149."""
import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar
from gpu_util import assert_same_codes, assert_same_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

TINY = np.float32(2.0 ** -149)
# block absmax in units of 2^-149: around the values where fl(m / Q) drops a
# whole unit below m / Q, and a few where the clamp does not bind
ABSMAX = {
    "int8": [190, 191, 253, 254, 300, 381, 1000, 127, 128, 64, 10, 1],
    "e4m3": [600, 671, 672, 896, 1000, 1343, 448, 449, 2000, 5],
    "int4": [10, 11, 13, 14, 20, 21, 7, 8, 3, 1],
}
Q = {"int8": 127.0, "e4m3": 448.0, "int4": 7.0}
CALLS = {
    "int8": (qar.qar_quantize_blocks, qar.qar_reduce_quantized, qar.qar_quantize_reduce, qar.qar_ring_step),
    "e4m3": (qar.qar_quantize_blocks_e4m3, qar.qar_reduce_quantized_e4m3, qar.qar_quantize_reduce_e4m3,
             qar.qar_ring_step_e4m3),
    "int4": (qar.qar_quantize_blocks_int4, qar.qar_reduce_quantized_int4, qar.qar_quantize_reduce_int4,
             qar.qar_ring_step_int4),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _data(seed, fmt, block, nb=80):
    rng = np.random.default_rng(seed)
    ks = ABSMAX[fmt]
    x = np.empty(nb * block, np.float32)
    for b in range(nb):
        k = ks[b % len(ks)]
        v = rng.integers(-k, k + 1, block)
        v[rng.integers(0, block)] = k if rng.integers(0, 2) else -k
        x[b * block:(b + 1) * block] = v.astype(np.float32) * TINY
    return x


def _oracle(o, fmt):
    if fmt == "int8":
        return o.quantize, lambda c, s, b, n: o.reduce(c, s, b), o.ring_step
    if fmt == "e4m3":
        return o.quantize_e4m3, lambda c, s, b, n: o.reduce_e4m3(c, s, b), o.ring_step_e4m3
    return o.quantize_int4, o.reduce_int4, o.ring_step_int4


def _bytes(t):
    return to_host(t).view(np.uint8)


@pytest.mark.parametrize("block", [64, 128, 256])
@pytest.mark.parametrize("fmt", ["int8", "e4m3", "int4"])
def test_subnormal_scales_where_the_clamp_binds(oracle_lib, fmt, block):
    quantize, reduce, quantize_reduce, ring_step = CALLS[fmt]
    o_quantize, o_reduce, o_ring = _oracle(oracle_lib, fmt)
    x0, x1 = _data(block, fmt, block), _data(block + 1, fmt, block)
    n = x0.size
    # the data do reach the clamp: some element's quotient rounds beyond Q
    s = (np.abs(x0).reshape(-1, block).max(axis=1) / np.float32(Q[fmt])).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = x0.reshape(-1, block) / s[:, None]
    assert np.nanmax(np.abs(np.rint(quot[s > 0]))) > Q[fmt]
    say(f"clamp {fmt} B={block}")
    c0, s0 = quantize(to_dev(x0), block)
    c1, s1 = quantize(to_dev(x1), block)
    out = torch.empty(n, dtype=torch.float32, device="cuda:0")
    rc, rs = reduce([c0, c1], [s0, s1], block, out=out)
    own_c, own_s = torch.empty_like(c1), torch.empty_like(s1)
    qc, qs = quantize_reduce(to_dev(x1), 1, [c0, own_c], [s0, own_s], block)
    gc, gs = ring_step(c0, s0, to_dev(x1), block)
    torch.cuda.synchronize()
    w0, v0 = o_quantize(x0, block)
    w1, v1 = o_quantize(x1, block)
    assert_same_codes(_bytes(c0), w0.view(np.uint8), "rank 0 codes")
    assert_same_f32(to_host(s0), v0, "rank 0 scales")
    assert_same_codes(_bytes(c1), w1.view(np.uint8), "rank 1 codes")
    wr, vr = o_reduce([w0, w1], [v0, v1], block, n)
    assert_same_codes(_bytes(rc), wr.view(np.uint8), "reduce codes")
    assert_same_f32(to_host(rs), vr, "reduce scales")
    if fmt == "int8":
        want_out = oracle_lib.dequantize(wr, vr, block, "f32")
    elif fmt == "e4m3":
        want_out = oracle_lib.dequantize_e4m3(wr, vr, block, "f32")
    else:
        want_out = oracle_lib.dequantize_int4(wr, vr, block, n, "f32")
    assert_same_f32(to_host(out), want_out, "reduce fp32 out")
    assert_same_codes(_bytes(own_c), w1.view(np.uint8), "step: own codes")
    assert_same_codes(_bytes(qc), wr.view(np.uint8), "step: codes")
    assert_same_f32(to_host(qs), vr, "step: scales")
    wg, vg = o_ring(w0, v0, x1, block)
    assert_same_codes(_bytes(gc), wg.view(np.uint8), "ring codes")
    assert_same_f32(to_host(gs), vg, "ring scales")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["int8", "e4m3", "int4"])
def test_fast_path_quotients_just_above_q(oracle_lib, fmt, dtype):
    """Normal block scales whose absmax element has a rounded quotient just
    above Q (fl(m / fl(m / Q)) = the next binary32 value after Q): the fast
    path takes no clamp, so the rounding to an integer (int8, 4-bit) or the
    E4M3 conversion (448 + 2^-15 must give 448) has to land on Q.  Blocks
    are picked from seeded absmax values by that property and checked
    against the oracle."""
    from block_wise_int8_amd import synth
    block = 64
    rng = np.random.default_rng(7)
    m = (rng.uniform(1, 2, 400_000) * np.exp2(rng.integers(-80, 120, 400_000))).astype(np.float32)
    if dtype == "bf16":
        m = (m.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    q = np.float32(Q[fmt])
    hit = m[(m / (m / q)) > q][:96]
    assert hit.size == 96
    x = (rng.uniform(-1, 1, (hit.size, block)) * hit[:, None]).astype(np.float32)
    pos = rng.integers(0, block, hit.size)
    x[np.arange(hit.size), pos] = np.where(rng.random(hit.size) < 0.5, hit, -hit)
    x = x.reshape(-1)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    quantize = CALLS[fmt][0]
    o_quantize = _oracle(oracle_lib, fmt)[0]
    say(f"fast-path quotient above Q: {fmt} {dtype}")
    c, s = quantize(to_dev(x), block)
    torch.cuda.synchronize()
    wc, ws = o_quantize(x, block)
    assert_same_codes(_bytes(c), wc.view(np.uint8), "codes")
    assert_same_f32(to_host(s), ws, "scales")
