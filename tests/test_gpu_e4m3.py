"""The FP8 E4M3 calls against the CPU oracle, element by element, through
the C ABI: codes (bytes), scales and dequantized values bit for bit.

The hardware conversion (v_cvt_pk_fp8_f32; a clamp to +-448 first on the
IEEE-division path, scales below 2^-90) is
checked at every rounding boundary of the format: for scales that are powers
of two the quotient is exact, so blocks can place it on every midpoint
between neighbouring E4M3 values, one ulp either side, and on the values
themselves, in both signs, subnormals included."""
import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth
from gpu_util import (SUM_OUTLIER, assert_same_bits16, assert_same_codes, assert_same_f32, mixed_bf16, mixed_f32,
                      ragged_n, say, to_dev, to_host)
from oracle import bounds

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _codes(t: torch.Tensor) -> np.ndarray:
    return to_host(t).view(np.uint8)


def _e4m3_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values in code order (from the
    oracle, which is pinned to torch's float8_e4m3fn)."""
    import oracle
    return oracle.load().e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)


# ----------------------------------------------------------------------------
# quantize


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_e4m3_parity(oracle_lib, dtype, block):
    n = ragged_n(block)
    x = mixed_bf16(block + 1, n, block) if dtype == "bf16" else mixed_f32(block + 1, n, block)
    say(f"e4m3 quantize {dtype} B={block} n={n}")
    codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(x), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_e4m3(x, block)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_codes(codes), wc, "E4M3 codes")


def test_quantize_e4m3_every_rounding_boundary(oracle_lib):
    """Blocks of 64 with absmax 448 * 2^k (scale exactly 2^k): quotients on
    every E4M3 value, every midpoint and the float32 neighbours of each
    midpoint, both signs, for k across the binary32 range."""
    v = _e4m3_values()
    mid = (v[:-1] + v[1:]) / 2
    q = np.concatenate([v, mid, np.nextafter(mid.astype(np.float32), np.float32(0)),
                        np.nextafter(mid.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    q = np.concatenate([q, -q, np.float32([0.0, -0.0, 2.0 ** -12, -2.0 ** -12, 2.0 ** -149, -2.0 ** -149])])
    q = q[np.abs(q) <= 448.0]
    per = 63
    q = np.concatenate([q, np.zeros((-q.size) % per, np.float32)]).reshape(-1, per)
    blocks = []
    for k in (-120, -60, -9, -1, 0, 3, 40, 100, 118):
        p = np.float32(2.0 ** k)
        blk = np.concatenate([np.full((q.shape[0], 1), np.float32(448.0) * p), q * p], axis=1)
        blocks.append(blk.astype(np.float32))
    x = np.concatenate(blocks).reshape(-1)
    say(f"e4m3 rounding boundaries n={x.size}")
    codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(x), 64)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_e4m3(x, 64)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_codes(codes), wc, "E4M3 codes at rounding boundaries")


def test_quantize_e4m3_every_fp32_rounding_class(oracle_lib):
    """Blocks led by 448 have scale 1, so the quotient is x itself: every
    binary32 exponent up to 448's, both signs, each value of the top 4
    mantissa bits (the 3 an E4M3 value keeps and the rounding bit), with
    the 19 bits below zero, lowest set, all set, or random."""
    rng = np.random.default_rng(97)
    e = np.arange(0, 136, dtype=np.uint32)[:, None, None]          # biased exponents of 0 .. 2^8
    top = np.arange(16, dtype=np.uint32)[None, :, None]
    low = np.stack([np.zeros(136 * 16, np.uint32), np.ones(136 * 16, np.uint32),
                    np.full(136 * 16, (1 << 19) - 1, np.uint32),
                    rng.integers(0, 1 << 19, 136 * 16).astype(np.uint32)], axis=1).reshape(136, 16, 4)
    bits = (e << 23) | (top << 19) | low
    bits = np.concatenate([bits.reshape(-1), bits.reshape(-1) | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    x = x[np.abs(x) <= 448.0]
    per = 63
    x = np.concatenate([x, np.zeros((-x.size) % per, np.float32)]).reshape(-1, per)
    x = np.concatenate([np.full((x.shape[0], 1), np.float32(448.0)), x], axis=1).reshape(-1)
    say(f"e4m3 fp32 rounding classes n={x.size}")
    codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(x), 64)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_e4m3(x, 64)
    assert np.all(ws == 1.0)
    assert_same_codes(_codes(codes), wc, "E4M3 codes of every fp32 rounding class")


def test_quantize_e4m3_every_bf16_against_many_scales(oracle_lib):
    """Every finite bf16 x against 128 absmax values spread over the bf16
    range (inexact scales, so the quotient's rounding matters too)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]
    v = (h.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(91)
    pos = h[(h > 0) & (h < 0x7F80)]
    picks = np.concatenate([rng.choice(pos, 122, replace=False),
                            np.uint16([0x0001, 0x0080, 0x3F80, 0x43E0, 0x7F7F, 0x0400])])
    blocks = []
    for a in picks:
        av = (np.uint32(a) << 16).view(np.float32)
        sel = h[np.abs(v) <= av]
        k = -(-sel.size // 255)
        sel = np.concatenate([sel, np.zeros(k * 255 - sel.size, np.uint16)]).reshape(k, 255)
        blocks.append(np.concatenate([np.full((k, 1), a, np.uint16), sel], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    say(f"e4m3 exhaustive bf16 grid n={x.size}")
    codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(x), 256)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_e4m3(x, 256)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_codes(codes), wc, "E4M3 codes")


def test_quantize_e4m3_random_scales(oracle_lib):
    """fp32 values of every magnitude against 4096 random scales, including
    scales below 2^-90 (the IEEE-division path) and subnormal ones."""
    rng = np.random.default_rng(93)
    nb = 4096
    e = rng.uniform(-149, 127, nb)
    amax = np.exp2(e).astype(np.float32)
    amax[amax == 0] = np.float32(2.0 ** -149)
    frac = rng.uniform(-1, 1, (nb, 63)) * np.exp2(-rng.uniform(0, 14, (nb, 63)))
    x = np.concatenate([amax[:, None], (frac * amax[:, None]).astype(np.float32)], axis=1).astype(np.float32)
    x = x.reshape(-1)
    say(f"e4m3 random scales n={x.size}")
    codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(x), 64)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_e4m3(x, 64)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_codes(codes), wc, "E4M3 codes")


# ----------------------------------------------------------------------------
# dequantize


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_e4m3_every_code(oracle_lib, out, block):
    """All 254 finite codes against scales across the range."""
    n = ragged_n(block)
    rng = np.random.default_rng(95 + block)
    codes = rng.integers(0, 256, n).astype(np.uint8)
    codes[:256] = np.arange(256, dtype=np.uint8)
    codes[np.isin(codes, [0x7F, 0xFF])] = 0x80
    nb = n // block
    scales = np.exp2(rng.uniform(-149, 119, nb)).astype(np.float32)
    scales[0] = 0.0
    scales[1] = np.float32(2.0 ** -149)
    say(f"e4m3 dequantize {out} B={block}")
    y = qar.qar_dequantize_e4m3(to_dev(codes), to_dev(scales), block,
                                out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    want = oracle_lib.dequantize_e4m3(codes, scales, block, out)
    if out == "bf16":
        assert_same_bits16(to_host(y), want, "dequantized bf16")
    else:
        assert_same_f32(to_host(y), want, "dequantized f32")


# ----------------------------------------------------------------------------
# reduce, one-kernel step, ring


def _ranks(o, xs, block):
    qs = [o.quantize_e4m3(x, block) for x in xs]
    return [q[0] for q in qs], [q[1] for q in qs]


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("nranks", [1, 2, 3, 8, 9, 32])
def test_reduce_e4m3_parity(oracle_lib, nranks, block):
    n = ragged_n(block, tiles=2)
    xs = [mixed_bf16(500 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _ranks(oracle_lib, xs, block)
    say(f"e4m3 reduce N={nranks} B={block} n={n}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    out16 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    oc, os_ = qar.qar_reduce_quantized_e4m3(dc, ds, block, out=out16)
    out32 = torch.empty(n, dtype=torch.float32, device="cuda:0")
    oc2, os2 = qar.qar_reduce_quantized_e4m3(dc, ds, block, out=out32)
    oc3, os3 = qar.qar_reduce_quantized_e4m3(dc, ds, block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce_e4m3(codes, scales, block)
    for c, s in ((oc, os_), (oc2, os2), (oc3, os3)):
        assert_same_codes(_codes(c), wc, "E4M3 reduce codes")
        assert_same_f32(to_host(s), ws, "E4M3 reduce scales")
    assert_same_bits16(to_host(out16), oracle_lib.dequantize_e4m3(wc, ws, block, "bf16"), "fused bf16 out")
    assert_same_f32(to_host(out32), oracle_lib.dequantize_e4m3(wc, ws, block, "f32"), "fused fp32 out")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nranks,own", [(1, 0), (4, 3), (8, 0), (9, 5)])
def test_quantize_reduce_e4m3_parity(oracle_lib, nranks, own, dtype):
    block = 128
    n = ragged_n(block, tiles=2)
    make = mixed_bf16 if dtype == "bf16" else mixed_f32
    xs = [make(700 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _ranks(oracle_lib, xs, block)
    say(f"e4m3 quantize_reduce N={nranks} own={own} {dtype}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[own].fill_(0x55)
    ds[own].fill_(-1.0)
    out = torch.empty(n, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = qar.qar_quantize_reduce_e4m3(to_dev(xs[own]), own, dc, ds, block, out=out)
    torch.cuda.synchronize()
    assert_same_codes(_codes(dc[own]), codes[own], "own codes")
    assert_same_f32(to_host(ds[own]), scales[own], "own scales")
    wc, ws = oracle_lib.reduce_e4m3(codes, scales, block)
    assert_same_codes(_codes(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    want = oracle_lib.dequantize_e4m3(wc, ws, block, dtype)
    if dtype == "bf16":
        assert_same_bits16(to_host(out), want, "out")
    else:
        assert_same_f32(to_host(out), want, "out")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_step_e4m3_parity(oracle_lib, dtype, block, in_place):
    n = ragged_n(block)
    make = mixed_bf16 if dtype == "bf16" else mixed_f32
    x0, x1 = make(11 + block, n, block, SUM_OUTLIER), make(12 + block, n, block, SUM_OUTLIER)
    c0, s0 = oracle_lib.quantize_e4m3(x0, block)
    say(f"e4m3 ring {dtype} B={block} in_place={in_place}")
    dc, ds = to_dev(c0), to_dev(s0)
    if in_place:
        oc, os_ = qar.qar_ring_step_e4m3(dc, ds, to_dev(x1), block, codes_out=dc, scales_out=ds)
    else:
        oc, os_ = qar.qar_ring_step_e4m3(dc, ds, to_dev(x1), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.ring_step_e4m3(c0, s0, x1, block)
    assert_same_codes(_codes(oc), wc, "E4M3 ring codes")
    assert_same_f32(to_host(os_), ws, "E4M3 ring scales")


# ----------------------------------------------------------------------------
# full-size workloads


@pytest.mark.parametrize("key", ["outliers", "prefill"])
def test_e4m3_workload(oracle_lib, key):
    """The outlier and prefill workloads with E4M3 codes: quantize of every
    rank, the one-kernel step with rank 0's raw data, all bit-exact; and the
    error against the exact sum within (3) with (1e) on sampled blocks."""
    w = synth.WORKLOADS[key]
    say(f"e4m3 {key}: generating {w.nranks} x {w.n}")
    host = synth.ranks(w)
    B = w.block
    dc, ds, oc, os_ = [], [], [], []
    for r, x in enumerate(host):
        c, s = qar.qar_quantize_blocks_e4m3(to_dev(x), B)
        torch.cuda.synchronize()
        wc, ws = oracle_lib.quantize_e4m3(x, B)
        assert_same_codes(_codes(c), wc, f"{key} rank {r} E4M3 codes")
        assert_same_f32(to_host(s), ws, f"{key} rank {r} scales")
        dc.append(c), ds.append(s), oc.append(wc), os_.append(ws)
    say(f"e4m3 {key}: quantize bit-exact")
    own_c, own_s = torch.empty_like(dc[0]), torch.empty_like(ds[0])
    out = torch.empty(w.n, dtype=torch.bfloat16, device="cuda:0")
    rc, rs = qar.qar_quantize_reduce_e4m3(to_dev(host[0]), 0, [own_c] + dc[1:], [own_s] + ds[1:], B, out=out)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce_e4m3(oc, os_, B)
    assert_same_codes(_codes(own_c), oc[0], f"{key} own codes")
    assert_same_codes(_codes(rc), wc, f"{key} reduce codes")
    assert_same_f32(to_host(rs), ws, f"{key} reduce scales")
    assert_same_bits16(to_host(out), oracle_lib.dequantize_e4m3(wc, ws, B, "bf16"), f"{key} out")
    say(f"e4m3 {key}: one-kernel step bit-exact")
    nb = w.n // B
    rng = np.random.default_rng(5)
    picks = np.unique(np.concatenate([rng.choice(nb, 2048, replace=False), [0, nb - 1]]))
    idx = (picks[:, None] * B + np.arange(B)).reshape(-1)
    xs = [(x[idx].astype(np.uint32) << 16).view(np.float32).astype(np.float64) for x in host]
    exact = np.sum(xs, axis=0)
    ys = [oracle_lib.dequantize_e4m3(c[idx], s[picks], B, "f32") for c, s in zip(oc, os_)]
    deq = oracle_lib.dequantize_e4m3(wc[idx], ws[picks], B, "f32").astype(np.float64)
    bnd = bounds.oneshot_bound_e4m3(xs, [s[picks] for s in os_], ys, ws[picks], B)
    err = np.abs(deq - exact)
    assert np.all(err <= bnd), f"{key}: E4M3 bound violated, worst ratio {np.max(err / bnd)}"
    say(f"e4m3 {key}: max err/bound {np.max(err / bnd):.3f}")


def test_e4m3_beyond_2_pow_31_elements(oracle_lib):
    """E4M3 quantize, dequantize and the one-kernel step (N = 2) at n above
    2**31, checked against the oracle on sampled blocks and the last ones."""
    from gpu_util import TILE
    block = 256
    n = (1 << 31) + 3 * TILE + 7 * block
    say(f"e4m3 large n={n}")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(77)
    x0 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 1.0, generator=g)
    x1 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 2.0, generator=g)
    c1, s1 = qar.qar_quantize_blocks_e4m3(x1, block)
    y1 = qar.qar_dequantize_e4m3(c1, s1, block, out_dtype=torch.bfloat16)
    c0 = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    s0 = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    fc, fs = qar.qar_quantize_reduce_e4m3(x0, 0, [c0, c1], [s0, s1], block)
    torch.cuda.synchronize()
    nb = n // block
    rng = np.random.default_rng(8)
    picks = np.concatenate([rng.choice(nb, 2000, replace=False), np.arange(nb - 40, nb)])
    pk = torch.from_numpy(picks).cuda()
    idx = torch.from_numpy((picks[:, None] * block + np.arange(block)).reshape(-1)).cuda()
    q = [oracle_lib.quantize_e4m3(to_host(x[idx]), block) for x in (x0, x1)]
    assert_same_codes(_codes(c1[idx]), q[1][0], "codes")
    assert_same_f32(to_host(s1[pk]), q[1][1], "scales")
    assert_same_bits16(to_host(y1[idx]), oracle_lib.dequantize_e4m3(q[1][0], q[1][1], block, "bf16"), "dequantized")
    wc, ws = oracle_lib.reduce_e4m3([a for a, _ in q], [b for _, b in q], block)
    assert_same_codes(_codes(c0[idx]), q[0][0], "own codes")
    assert_same_codes(_codes(fc[idx]), wc, "step codes")
    assert_same_f32(to_host(fs[pk]), ws, "step scales")
    del x0, x1, c0, c1, s0, s1, y1, fc, fs
    torch.cuda.empty_cache()


def test_golden_e4m3_cases_on_gpu():
    """The hand-derived E4M3 cases through the C ABI."""
    import golden_cases as gc
    g = gc.load_e4m3()
    B = g["block"]
    for case in g["quantize"]:
        say(f"e4m3 golden: {case['name']}")
        codes, scales = qar.qar_quantize_blocks_e4m3(to_dev(gc.e4m3_x(case, B)), B)
        y = qar.qar_dequantize_e4m3(codes, scales, B, out_dtype=torch.float32)
        torch.cuda.synchronize()
        want = gc.e4m3_bytes(case["codes"])
        assert list(_codes(codes)[:len(want)]) == want, case["name"]
        assert to_host(scales).view(np.uint32)[0] == np.float32(gc.e4m3_scale(case)).view(np.uint32), case["name"]
        assert list(to_host(y).view(np.uint32)[:len(want)]) == gc.e4m3_dequant_bits(case), case["name"]
    for case in g["reduce"]:
        q = [qar.qar_quantize_blocks_e4m3(to_dev(gc.pad(r, B)), B) for r in case["ranks"]]
        oc, os_ = qar.qar_reduce_quantized_e4m3([c for c, _ in q], [s for _, s in q], B)
        torch.cuda.synchronize()
        assert list(_codes(oc)[:len(case["codes"])]) == gc.e4m3_bytes(case["codes"]), case["name"]
        assert to_host(os_)[0] == np.float32(case["scale"]), case["name"]
    for case in g["ring_step"]:
        c = to_dev(gc.pad(gc.e4m3_bytes(case["codes_in"]), B, np.uint8))
        oc, os_ = qar.qar_ring_step_e4m3(c, to_dev(np.float32([case["scale_in"]])), to_dev(gc.pad(case["local"], B)), B)
        torch.cuda.synchronize()
        assert list(_codes(oc)[:len(case["codes"])]) == gc.e4m3_bytes(case["codes"]), case["name"]
        assert to_host(os_)[0] == np.float32(case["scale"]), case["name"]
