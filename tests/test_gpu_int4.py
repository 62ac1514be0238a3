"""The 4-bit calls (two codes per byte) against the CPU oracle, through the
C ABI: packed code bytes, scales and dequantized values bit for bit."""
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


def _packed(t: torch.Tensor) -> np.ndarray:
    return to_host(t).view(np.uint8)


def _same_out(got, want, kind, what):
    if kind == "bf16":
        assert_same_bits16(got, want, what)
    else:
        assert_same_f32(got, want, what)


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_int4_parity(oracle_lib, dtype, block):
    n = ragged_n(block)
    x = mixed_bf16(block + 7, n, block) if dtype == "bf16" else mixed_f32(block + 7, n, block)
    say(f"int4 quantize {dtype} B={block} n={n}")
    codes, scales = qar.qar_quantize_blocks_int4(to_dev(x), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_int4(x, block)
    assert codes.numel() == n // 2
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_packed(codes), wc, "packed 4-bit codes")


def test_quantize_int4_every_bf16_against_many_scales(oracle_lib):
    """Every finite bf16 x against 128 absmax values (blocks of 256)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]
    v = (h.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(111)
    pos = h[(h > 0) & (h < 0x7F80)]
    picks = np.concatenate([rng.choice(pos, 124, replace=False), np.uint16([0x0001, 0x0080, 0x40E0, 0x7F7F])])
    blocks = []
    for a in picks:
        av = (np.uint32(a) << 16).view(np.float32)
        sel = h[np.abs(v) <= av]
        k = -(-sel.size // 255)
        sel = np.concatenate([sel, np.zeros(k * 255 - sel.size, np.uint16)]).reshape(k, 255)
        blocks.append(np.concatenate([np.full((k, 1), a, np.uint16), sel], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    say(f"int4 exhaustive bf16 grid n={x.size}")
    codes, scales = qar.qar_quantize_blocks_int4(to_dev(x), 256)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_int4(x, 256)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_packed(codes), wc, "packed 4-bit codes")


def test_quantize_int4_near_ties(oracle_lib):
    """Quotients within a few ulps of every half-integer -6.5 .. 6.5."""
    rng = np.random.default_rng(113)
    nb = 2048
    amax = np.exp(rng.uniform(-60, 60, nb)).astype(np.float32)
    s = (amax / np.float32(7.0)).astype(np.float32)
    k = rng.integers(-7, 7, (nb, 63)) + 0.5
    base = (k * s.astype(np.float64)[:, None]).astype(np.float32)
    x = (base.view(np.int32) + rng.integers(-3, 4, (nb, 63)).astype(np.int32)).view(np.float32)
    x = np.where(np.abs(x) <= amax[:, None], x, base)
    x = np.concatenate([amax[:, None], x], axis=1).astype(np.float32).reshape(-1)
    codes, scales = qar.qar_quantize_blocks_int4(to_dev(x), 64)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize_int4(x, 64)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(_packed(codes), wc, "packed 4-bit codes")


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_int4_parity(oracle_lib, out, block):
    """Every byte value (both nibbles, -8 included) against scales across
    the range."""
    n = ragged_n(block)
    rng = np.random.default_rng(115 + block)
    packed = rng.integers(0, 256, n // 2).astype(np.uint8)
    packed[:256] = np.arange(256, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-149, 124, n // block)).astype(np.float32)
    scales[0] = 0.0
    # both sides of 2^123, where the kernels' code-to-float conversion changes
    scales[1:4] = np.float32(2.0 ** 123), np.nextafter(np.float32(2.0 ** 123), np.float32(np.inf)), \
        np.float32(2.0 ** 123.99)
    y = qar.qar_dequantize_int4(to_dev(packed), to_dev(scales), block,
                                out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    _same_out(to_host(y), oracle_lib.dequantize_int4(packed, scales, block, n, out), out, "dequantized")


@pytest.mark.parametrize("nranks", [1, 2])
def test_reduce_int4_every_byte_every_scale_range(oracle_lib, nranks):
    """Arbitrary packed bytes (all 256 values, so -8 too) reduced with scales
    from the subnormal range up to 2^124-2^125 (both sides of 2^123, where
    the kernels' code-to-float conversion changes), zero and tiny scales
    included; the sums stay finite."""
    block = 64
    n = ragged_n(block)
    rng = np.random.default_rng(4242 + nranks)
    top = 125 if nranks == 1 else 124
    codes, scales = [], []
    for r in range(nranks):
        packed = rng.integers(0, 256, n // 2).astype(np.uint8)
        packed[:256] = np.arange(256, dtype=np.uint8)
        sc = np.exp2(rng.uniform(-149, top, n // block)).astype(np.float32)
        sc[rng.integers(0, n // block, 8)] = 0.0
        sc[:4] = np.float32(2.0 ** 123), np.nextafter(np.float32(2.0 ** 123), np.float32(np.inf)), \
            np.float32(2.0 ** (top - 0.01)), np.float32(2.0 ** -149)
        codes.append(packed)
        scales.append(sc)
    say(f"int4 reduce every byte N={nranks}")
    out = torch.empty(n, dtype=torch.float32, device="cuda:0")
    out16 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    oc, os_ = qar.qar_reduce_quantized_int4(dc, ds, block, out=out)
    oc16, os16 = qar.qar_reduce_quantized_int4(dc, ds, block, out=out16)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce_int4(codes, scales, block, n)
    assert float(ws.max()) > 2.0 ** 123                 # the fused output's slow widening runs too
    assert_same_codes(_packed(oc), wc, "packed codes")
    assert_same_f32(to_host(os_), ws, "scales")
    assert_same_f32(to_host(out), oracle_lib.dequantize_int4(wc, ws, block, n, "f32"), "fp32 out")
    assert_same_codes(_packed(oc16), wc, "packed codes (bf16 out)")
    assert_same_bits16(to_host(out16), oracle_lib.dequantize_int4(wc, ws, block, n, "bf16"), "bf16 out")


def _ranks(o, xs, block):
    qs = [o.quantize_int4(x, block) for x in xs]
    return [q[0] for q in qs], [q[1] for q in qs]


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("nranks", [1, 2, 3, 8, 9, 32])
def test_reduce_int4_parity(oracle_lib, nranks, block):
    n = ragged_n(block, tiles=2)
    xs = [mixed_bf16(900 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _ranks(oracle_lib, xs, block)
    say(f"int4 reduce N={nranks} B={block}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    out16 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    oc, os_ = qar.qar_reduce_quantized_int4(dc, ds, block, out=out16)
    out32 = torch.empty(n, dtype=torch.float32, device="cuda:0")
    oc2, os2 = qar.qar_reduce_quantized_int4(dc, ds, block, out=out32)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce_int4(codes, scales, block, n)
    for c, s in ((oc, os_), (oc2, os2)):
        assert_same_codes(_packed(c), wc, "packed codes")
        assert_same_f32(to_host(s), ws, "scales")
    assert_same_bits16(to_host(out16), oracle_lib.dequantize_int4(wc, ws, block, n, "bf16"), "bf16 out")
    assert_same_f32(to_host(out32), oracle_lib.dequantize_int4(wc, ws, block, n, "f32"), "fp32 out")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nranks,own", [(1, 0), (4, 2), (8, 7), (9, 0)])
def test_quantize_reduce_int4_parity(oracle_lib, nranks, own, dtype):
    block = 256
    n = ragged_n(block, tiles=2)
    make = mixed_bf16 if dtype == "bf16" else mixed_f32
    xs = [make(1300 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _ranks(oracle_lib, xs, block)
    say(f"int4 quantize_reduce N={nranks} own={own} {dtype}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[own].fill_(0x55)
    ds[own].fill_(-1.0)
    out = torch.empty(n, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = qar.qar_quantize_reduce_int4(to_dev(xs[own]), own, dc, ds, block, out=out)
    torch.cuda.synchronize()
    assert_same_codes(_packed(dc[own]), codes[own], "own codes")
    assert_same_f32(to_host(ds[own]), scales[own], "own scales")
    wc, ws = oracle_lib.reduce_int4(codes, scales, block, n)
    assert_same_codes(_packed(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    _same_out(to_host(out), oracle_lib.dequantize_int4(wc, ws, block, n, dtype), dtype, "out")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("outlier", [SUM_OUTLIER, 1.6e38])
def test_ring_step_int4_parity(oracle_lib, dtype, block, in_place, outlier):
    """The second outlier value gives scales above 2^123, where the kernels
    convert codes to float another way."""
    n = ragged_n(block)
    make = mixed_bf16 if dtype == "bf16" else mixed_f32
    x0, x1 = make(21 + block, n, block, outlier), make(22 + block, n, block, outlier)
    c0, s0 = oracle_lib.quantize_int4(x0, block)
    dc, ds = to_dev(c0), to_dev(s0)
    if in_place:
        oc, os_ = qar.qar_ring_step_int4(dc, ds, to_dev(x1), block, codes_out=dc, scales_out=ds)
    else:
        oc, os_ = qar.qar_ring_step_int4(dc, ds, to_dev(x1), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.ring_step_int4(c0, s0, x1, block)
    assert_same_codes(_packed(oc), wc, "ring codes")
    assert_same_f32(to_host(os_), ws, "ring scales")


@pytest.mark.parametrize("key", ["outliers", "prefill"])
def test_int4_workload(oracle_lib, key):
    """The outlier and prefill workloads with 4-bit codes: quantize of every
    rank and the one-kernel step, bit-exact; error within bound (3) on
    sampled blocks."""
    w = synth.WORKLOADS[key]
    say(f"int4 {key}: generating {w.nranks} x {w.n}")
    host = synth.ranks(w)
    B = w.block
    dc, ds, oc, os_ = [], [], [], []
    for r, x in enumerate(host):
        c, s = qar.qar_quantize_blocks_int4(to_dev(x), B)
        torch.cuda.synchronize()
        wc, ws = oracle_lib.quantize_int4(x, B)
        assert_same_codes(_packed(c), wc, f"{key} rank {r} codes")
        assert_same_f32(to_host(s), ws, f"{key} rank {r} scales")
        dc.append(c), ds.append(s), oc.append(wc), os_.append(ws)
    own_c, own_s = torch.empty_like(dc[0]), torch.empty_like(ds[0])
    out = torch.empty(w.n, dtype=torch.bfloat16, device="cuda:0")
    rc, rs = qar.qar_quantize_reduce_int4(to_dev(host[0]), 0, [own_c] + dc[1:], [own_s] + ds[1:], B, out=out)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce_int4(oc, os_, B, w.n)
    assert_same_codes(_packed(own_c), oc[0], f"{key} own codes")
    assert_same_codes(_packed(rc), wc, f"{key} reduce codes")
    assert_same_f32(to_host(rs), ws, f"{key} reduce scales")
    assert_same_bits16(to_host(out), oracle_lib.dequantize_int4(wc, ws, B, w.n, "bf16"), f"{key} out")
    nb = w.n // B
    rng = np.random.default_rng(9)
    picks = np.unique(np.concatenate([rng.choice(nb, 2048, replace=False), [0, nb - 1]]))
    idx = (picks[:, None] * B + np.arange(B)).reshape(-1)
    bidx = (picks[:, None] * (B // 2) + np.arange(B // 2)).reshape(-1)
    n_s = idx.size
    xs = [(x[idx].astype(np.uint32) << 16).view(np.float32).astype(np.float64) for x in host]
    exact = np.sum(xs, axis=0)
    ys = [oracle_lib.dequantize_int4(c[bidx], s[picks], B, n_s, "f32") for c, s in zip(oc, os_)]
    deq = oracle_lib.dequantize_int4(wc[bidx], ws[picks], B, n_s, "f32").astype(np.float64)
    bnd = bounds.oneshot_bound(xs, [s[picks] for s in os_], ys, ws[picks], B)
    err = np.abs(deq - exact)
    assert np.all(err <= bnd), f"{key}: 4-bit bound violated, worst ratio {np.max(err / bnd)}"
    say(f"int4 {key}: bit-exact; max err/bound {np.max(err / bnd):.3f}")


def test_int4_beyond_2_pow_31_elements(oracle_lib):
    """4-bit quantize, dequantize, reduce and the one-kernel step (N = 2) at
    n above 2**31 (code buffers above 2**30 bytes), checked against the
    oracle on sampled blocks and the last ones."""
    from gpu_util import TILE
    block = 256
    n = (1 << 31) + 3 * TILE + 7 * block
    say(f"int4 large n={n}")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(79)
    x0 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 1.0, generator=g)
    x1 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 2.0, generator=g)
    c1, s1 = qar.qar_quantize_blocks_int4(x1, block)
    y1 = qar.qar_dequantize_int4(c1, s1, block, out_dtype=torch.bfloat16)
    c0 = torch.empty(n // 2, dtype=torch.uint8, device="cuda:0")
    s0 = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    fc, fs = qar.qar_quantize_reduce_int4(x0, 0, [c0, c1], [s0, s1], block)
    q0, qs0 = qar.qar_quantize_blocks_int4(x0, block)
    rc, rs = qar.qar_reduce_quantized_int4([q0, c1], [qs0, s1], block)
    torch.cuda.synchronize()
    nb = n // block
    rng = np.random.default_rng(9)
    picks = np.concatenate([rng.choice(nb, 2000, replace=False), np.arange(nb - 40, nb)])
    pk = torch.from_numpy(picks).cuda()
    idx = torch.from_numpy((picks[:, None] * block + np.arange(block)).reshape(-1)).cuda()
    cidx = torch.from_numpy((picks[:, None] * (block // 2) + np.arange(block // 2)).reshape(-1)).cuda()
    q = [oracle_lib.quantize_int4(to_host(x[idx]), block) for x in (x0, x1)]
    m = idx.numel()
    assert_same_codes(_packed(c1[cidx]), q[1][0], "codes")
    assert_same_f32(to_host(s1[pk]), q[1][1], "scales")
    assert_same_bits16(to_host(y1[idx]), oracle_lib.dequantize_int4(q[1][0], q[1][1], block, m, "bf16"),
                       "dequantized")
    wc, ws = oracle_lib.reduce_int4([a for a, _ in q], [b for _, b in q], block, m)
    assert_same_codes(_packed(c0[cidx]), q[0][0], "own codes")
    for c, s_, what in ((fc, fs, "step"), (rc, rs, "reduce")):
        assert_same_codes(_packed(c[cidx]), wc, f"{what} codes")
        assert_same_f32(to_host(s_[pk]), ws, f"{what} scales")
    del x0, x1, c0, c1, s0, s1, y1, fc, fs, q0, qs0, rc, rs
    torch.cuda.empty_cache()
