"""libqar's HIP kernels against the CPU oracle, element by element, through
the C ABI.  Codes and scales must match bit for bit, dequantized fp32 and
bf16 values too (the method fixes every rounding; there is no tolerance).

Sizes span several 4096-element tiles plus a ragged tail (n is a multiple
of the block but not of the tile)."""
import numpy as np
import pytest
import torch

import golden_cases as gc
from block_wise_int8_amd import qar, synth
from gpu_util import (SUM_OUTLIER, TILE, assert_same_bits16, assert_same_codes, assert_same_f32, f32_bits,
                      mixed_bf16, mixed_f32, oracle_allreduce, ragged_n, say, to_dev, to_host)

pytestmark = pytest.mark.gpu

CHUNK_RUN = qar.QAR_CHUNK_RUN_ELEMS      # elements per run of the chunked calls' interleaved chunks


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()
    torch.cuda.init()


# ----------------------------------------------------------------------------
# quantize


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_parity(oracle_lib, dtype, block):
    n = ragged_n(block)
    x = mixed_bf16(block, n, block) if dtype == "bf16" else mixed_f32(block, n, block)
    say(f"quantize {dtype} B={block} n={n}")
    codes, scales = qar.qar_quantize_blocks(to_dev(x), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize(x, block)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(to_host(codes), wc, "codes")


def test_quantize_every_bf16_against_many_scales(oracle_lib):
    """Every finite bf16 x against 256 absmax values spread over the bf16
    range: blocks of 256 holding the absmax and 255 values |x| <= absmax."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]
    v = (h.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(77)
    pos = h[(h > 0) & (h < 0x7F80)]
    picks = np.concatenate([rng.choice(pos, 248, replace=False),
                            np.uint16([0x0001, 0x0080, 0x3F80, 0x42FE, 0x7F7F, 0x3C01, 0x4300, 0x0400])])
    blocks = []
    for a in picks:
        av = (np.uint32(a) << 16).view(np.float32)
        sel = h[np.abs(v) <= av]
        k = -(-sel.size // 255)
        sel = np.concatenate([sel, np.zeros(k * 255 - sel.size, np.uint16)]).reshape(k, 255)
        blocks.append(np.concatenate([np.full((k, 1), a, np.uint16), sel], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    say(f"exhaustive bf16 grid n={x.size}")
    codes, scales = qar.qar_quantize_blocks(to_dev(x), 256)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize(x, 256)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(to_host(codes), wc, "codes")


def test_quantize_f32_near_ties(oracle_lib):
    """fp32 quotients within a few ulps of every half-integer, for 2048
    random scales: blocks of 64 = the absmax element + 63 near-tie values."""
    rng = np.random.default_rng(78)
    nb = 2048
    amax = np.exp(rng.uniform(-60, 60, nb)).astype(np.float32)
    s = (amax / np.float32(127.0)).astype(np.float32)
    k = rng.integers(-127, 127, (nb, 63)) + 0.5
    base = (k * s.astype(np.float64)[:, None]).astype(np.float32)
    nudge = rng.integers(-3, 4, (nb, 63)).astype(np.int32)
    x = (base.view(np.int32) + nudge).view(np.float32)
    x = np.where(np.abs(x) <= amax[:, None], x, base)
    x = np.concatenate([amax[:, None], x], axis=1).astype(np.float32).reshape(-1)
    say(f"near ties n={x.size}")
    codes, scales = qar.qar_quantize_blocks(to_dev(x), 64)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.quantize(x, 64)
    assert_same_f32(to_host(scales), ws, "scales")
    assert_same_codes(to_host(codes), wc, "codes")


# ----------------------------------------------------------------------------
# dequantize


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_parity(oracle_lib, out, block):
    n = ragged_n(block)
    rng = np.random.default_rng(block + 3)
    codes = rng.integers(-128, 128, n).astype(np.int8)
    scales = np.abs(synth.wide_range_f32(block + 4, n // block, 1, log2_span=110)).astype(np.float32)
    scales[:6] = np.float32([0.0, 2.0 ** -149, 2.0 ** -140, 1.0 / 127, 2.6e36, 1.0e36])
    say(f"dequantize {out} B={block} n={n}")
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    y = qar.qar_dequantize(to_dev(codes), to_dev(scales), block, out_dtype=dt)
    torch.cuda.synchronize()
    want = oracle_lib.dequantize(codes, scales, block, out)
    if out == "bf16":
        assert_same_bits16(to_host(y), want, "bf16 out")
    else:
        assert_same_f32(to_host(y), want, "fp32 out")


# ----------------------------------------------------------------------------
# reduce


def _rank_codes(oracle_lib, xs, block):
    qs = [oracle_lib.quantize(x, block) for x in xs]
    return [q[0] for q in qs], [q[1] for q in qs]


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("nranks", [1, 2, 3, 4, 7, 8, 9, 16, 32])
def test_reduce_parity(oracle_lib, nranks, block):
    n = ragged_n(block, tiles=2)
    xs = [mixed_bf16(100 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _rank_codes(oracle_lib, xs, block)
    say(f"reduce N={nranks} B={block} n={n}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    out16 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    oc, os_ = qar.qar_reduce_quantized(dc, ds, block, out=out16)
    out32 = torch.empty(n, dtype=torch.float32, device="cuda:0")
    oc2, os2 = qar.qar_reduce_quantized(dc, ds, block, out=out32)
    oc3, os3 = qar.qar_reduce_quantized(dc, ds, block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce(codes, scales, block)
    assert_same_f32(to_host(os_), ws, "scales")
    assert_same_codes(to_host(oc), wc, "codes")
    assert_same_bits16(to_host(out16), oracle_lib.dequantize(wc, ws, block, "bf16"), "fused bf16 out")
    assert_same_f32(to_host(out32), oracle_lib.dequantize(wc, ws, block, "f32"), "fused fp32 out")
    for c, s in ((oc2, os2), (oc3, os3)):
        assert_same_codes(to_host(c), wc, "codes (other out variant)")
        assert_same_f32(to_host(s), ws, "scales (other out variant)")


def test_reduce_in_place(oracle_lib):
    block, n, nranks = 256, ragged_n(256), 4
    xs = [mixed_bf16(900 + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _rank_codes(oracle_lib, xs, block)
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    say("reduce in place into rank 2")
    qar.qar_reduce_quantized(dc, ds, block, codes_out=dc[2], scales_out=ds[2])
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce(codes, scales, block)
    assert_same_codes(to_host(dc[2]), wc, "codes")
    assert_same_f32(to_host(ds[2]), ws, "scales")


@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nranks,own", [(1, 0), (3, 1), (8, 0), (8, 7), (9, 8), (32, 13)])
def test_quantize_reduce_parity(oracle_lib, nranks, own, dtype, block):
    """The fused call: rank own quantized from its raw data in the same pass
    as the reduce.  Its codes and scales, and the result, equal the oracle's
    quantize followed by its reduce."""
    n = ragged_n(block, tiles=2)
    make = mixed_bf16 if dtype == "bf16" else mixed_f32
    xs = [make(300 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _rank_codes(oracle_lib, xs, block)
    say(f"quantize_reduce N={nranks} own={own} {dtype} B={block} n={n}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[own].fill_(0x55)                      # written by the call
    ds[own].fill_(-1.0)
    out = torch.empty(n, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = qar.qar_quantize_reduce(to_dev(xs[own]), own, dc, ds, block, out=out)
    oc2, os2 = qar.qar_quantize_reduce(to_dev(xs[own]), own, dc, ds, block)
    torch.cuda.synchronize()
    assert_same_codes(to_host(dc[own]), codes[own], "own codes")
    assert_same_f32(to_host(ds[own]), scales[own], "own scales")
    wc, ws = oracle_lib.reduce(codes, scales, block)
    for c, s in ((oc, os_), (oc2, os2)):
        assert_same_codes(to_host(c), wc, "codes")
        assert_same_f32(to_host(s), ws, "scales")
    want = oracle_lib.dequantize(wc, ws, block, dtype)
    if dtype == "bf16":
        assert_same_bits16(to_host(out), want, "fused out")
    else:
        assert_same_f32(to_host(out), want, "fused out")


@pytest.mark.parametrize("nstreams", [1, 4])
@pytest.mark.parametrize("nchunks", [1, 3, 8, 16, 32, 64])
def test_pipelined_bit_identical(oracle_lib, nchunks, nstreams):
    # chunks are interleaved runs of 2^18 elements: five and a part here
    block, nranks = 64, 5
    n = 5 * CHUNK_RUN + ragged_n(block, tiles=3)
    xs = [mixed_f32(700 + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _rank_codes(oracle_lib, xs, block)
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    out = torch.empty(n, dtype=torch.float32, device="cuda:0")
    say(f"pipelined nchunks={nchunks} nstreams={nstreams}")
    oc, os_ = qar.qar_reduce_quantized_pipelined(dc, ds, block, nchunks, streams, out=out)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce(codes, scales, block)
    assert_same_codes(to_host(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    assert_same_f32(to_host(out), oracle_lib.dequantize(wc, ws, block, "f32"), "out")


@pytest.mark.parametrize("nranks", [5, 16])
@pytest.mark.parametrize("with_caller", [False, True])
@pytest.mark.parametrize("nchunks,nstreams", [(1, 1), (3, 2), (8, 4), (16, 4), (5, 16)])
def test_chunked_bit_identical(oracle_lib, nchunks, nstreams, with_caller, nranks):
    """qar_reduce_quantized_chunked: chunk c (runs c, c + C, ... of 2^18
    elements) on streams[c % S] with no event of its own; the caller forks
    the streams off the current one, runs two calls back to back (the second
    reusing the first's output buffers, as a pipelined sequence of reduces
    does) and joins them.  n spans five runs and a ragged part of a sixth."""
    block = 64
    n = 5 * CHUNK_RUN + ragged_n(block, tiles=3)
    xs = [mixed_f32(710 + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    codes, scales = _rank_codes(oracle_lib, xs, block)
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    cur = torch.cuda.current_stream()
    streams = ([cur] if with_caller else []) + [torch.cuda.Stream() for _ in range(nstreams - with_caller)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    co = torch.empty(n, dtype=torch.int8, device="cuda:0")
    so = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    say(f"chunked nchunks={nchunks} nstreams={nstreams} with_caller={with_caller}")
    fork = torch.cuda.Event()
    fork.record(cur)
    for st in streams:
        st.wait_event(fork)
    qar.qar_reduce_quantized_chunked(dc[::-1], ds[::-1], block, nchunks, streams, co, so)   # overwritten next
    qar.qar_reduce_quantized_chunked(dc, ds, block, nchunks, streams, co, so, out=out)
    for st in streams:
        done = torch.cuda.Event()
        done.record(st)
        cur.wait_event(done)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.reduce(codes, scales, block)
    assert_same_codes(to_host(co), wc, "codes")
    assert_same_f32(to_host(so), ws, "scales")
    assert_same_bits16(to_host(out), oracle_lib.dequantize(wc, ws, block, "bf16"), "out")


def test_stale_runtime_error_does_not_fail_a_good_call():
    """A launch reports its own status: an error an unrelated HIP call left
    on the thread (an invalid hipSetDevice) must not turn a valid libqar
    call into QAR_ERR_HIP."""
    import ctypes
    # the HIP runtime this process already runs (torch's copy, which libqar
    # binds to by its soname), not another instance of it
    maps = open("/proc/self/maps").read().split()
    hip = ctypes.CDLL(next(p for p in maps if "libamdhip64.so" in p))
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    x = torch.ones(4096, dtype=torch.bfloat16, device="cuda:0")
    L = qar.lib()
    codes = torch.empty(4096, dtype=torch.int8, device="cuda:0")
    scales = torch.empty(16, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    # every tensor exists before the error is planted: torch checks the
    # thread's last error after its own launches
    assert hip.hipSetDevice(1 << 20) != 0                # hipErrorInvalidDevice, left on the thread
    st = L.qar_quantize_blocks(x.data_ptr(), qar.QAR_BF16, 4096, 256, codes.data_ptr(), scales.data_ptr(), stream)
    assert st == qar.QAR_OK, L.qar_last_error()
    hip.hipGetLastError()                                 # clear what the test left behind
    torch.cuda.synchronize()
    assert bool((codes == 127).all()) and bool((scales == 1.0 / 127).all())


# ----------------------------------------------------------------------------
# ring step


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("block", qar.BLOCK_SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_step_parity(oracle_lib, dtype, block, in_place):
    n = ragged_n(block)
    mk = mixed_bf16 if dtype == "bf16" else mixed_f32
    x0, x1 = mk(300 + block, n, block, SUM_OUTLIER), mk(301 + block, n, block, SUM_OUTLIER)
    c0, s0 = oracle_lib.quantize(x0, block)
    dc, ds = to_dev(c0), to_dev(s0)
    say(f"ring step {dtype} B={block} in_place={in_place}")
    if in_place:
        oc, os_ = qar.qar_ring_step(dc, ds, to_dev(x1), block, codes_out=dc, scales_out=ds)
    else:
        oc, os_ = qar.qar_ring_step(dc, ds, to_dev(x1), block)
    torch.cuda.synchronize()
    wc, ws = oracle_lib.ring_step(c0, s0, x1, block)
    assert_same_codes(to_host(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")


# ----------------------------------------------------------------------------
# the unquantized comparator


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nranks", [1, 2, 5, 8, 9, 16, 32])
def test_reduce_unquantized_parity(oracle_lib, nranks, dtype):
    n = 2 * TILE + 16 * 7
    mk = mixed_bf16 if dtype == "bf16" else mixed_f32
    xs = [mk(500 + nranks * 40 + r, n, 16, SUM_OUTLIER) for r in range(nranks)]
    say(f"unquantized reduce N={nranks} {dtype} n={n}")
    dx = [to_dev(x) for x in xs]
    out = qar.qar_reduce_unquantized(dx)
    qar.qar_reduce_unquantized(dx, out=dx[-1])                # in place into the last rank
    torch.cuda.synchronize()
    want = oracle_lib.reduce_unquantized(xs)
    if dtype == "bf16":
        assert_same_bits16(to_host(out), want, "sum")
        assert_same_bits16(to_host(dx[-1]), want, "sum in place")
    else:
        assert_same_f32(to_host(out), want, "sum")
        assert_same_f32(to_host(dx[-1]), want, "sum in place")


# ----------------------------------------------------------------------------
# the whole AllReduce on one GPU


@pytest.mark.parametrize("schedule", ["one_shot", "ring"])
@pytest.mark.parametrize("nranks,nchunks,nstreams,dtype,block", [
    (1, 2, 2, "bf16", 128), (2, 1, 1, "bf16", 256), (3, 3, 2, "bf16", 128), (4, 4, 4, "bf16", 256), (4, 16, 4, "f32", 64),
    (8, 8, 4, "bf16", 256), (5, 7, 3, "f32", 128)])
def test_allreduce_simulated(oracle_lib, schedule, nranks, nchunks, nstreams, dtype, block):
    n = ragged_n(block, tiles=3)
    mk = mixed_bf16 if dtype == "bf16" else mixed_f32
    xs = [mk(800 + 10 * nranks + r, n, block, SUM_OUTLIER) for r in range(nranks)]
    say(f"allreduce {schedule} N={nranks} chunks={nchunks} streams={nstreams} {dtype} B={block}")
    dx = [to_dev(x) for x in xs]
    nwork = nranks if schedule == "one_shot" else 1
    wc = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(nwork)]
    ws = [torch.empty(n // block, dtype=torch.float32, device="cuda:0") for _ in range(nwork)]
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    out = qar.qar_allreduce_simulated(dx, block, schedule, nchunks, streams, workspace=(wc, ws))
    torch.cuda.synchronize()
    c, s, y = oracle_allreduce(oracle_lib, xs, block, schedule, nchunks)
    assert_same_codes(to_host(wc[0]), c, "result codes")
    assert_same_f32(to_host(ws[0]), s, "result scales")
    if dtype == "bf16":
        assert_same_bits16(to_host(out), y, "result")
    else:
        assert_same_f32(to_host(out), y, "result")


# ----------------------------------------------------------------------------
# contract details


def test_concurrent_streams_and_repeat_runs(oracle_lib):
    """Two reduces on two streams at once, each repeated: every run equals
    the oracle (no shared state between calls, deterministic results)."""
    block, n = 256, ragged_n(256, tiles=8)
    jobs = []
    for k in range(2):
        xs = [mixed_bf16(1000 + 10 * k + r, n, block, SUM_OUTLIER) for r in range(4)]
        codes, scales = _rank_codes(oracle_lib, xs, block)
        jobs.append(([to_dev(c) for c in codes], [to_dev(s) for s in scales], oracle_lib.reduce(codes, scales, block)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()            # inputs were copied on the default stream
    for rep in range(3):
        for (dc, ds, _), st_ in zip(jobs, streams):
            outs.append(qar.qar_reduce_quantized(dc, ds, block, stream=st_))
    torch.cuda.synchronize()
    for i, (c, s) in enumerate(outs):
        wc, ws = jobs[i % 2][2]
        assert_same_codes(to_host(c), wc, f"run {i} codes")
        assert_same_f32(to_host(s), ws, f"run {i} scales")


def test_subrange_call_equals_slice(oracle_lib):
    """A block-aligned sub-range (offset pointers) is a valid call with the
    same results in that range."""
    block, n = 128, ragged_n(128)
    x = mixed_bf16(55, n, block)
    dx = to_dev(x)
    codes, scales = qar.qar_quantize_blocks(dx, block)
    k0, k1 = 7, n // block - 3
    sub_c, sub_s = qar.qar_quantize_blocks(dx[k0 * block:k1 * block], block)
    torch.cuda.synchronize()
    assert_same_codes(to_host(sub_c), to_host(codes)[k0 * block:k1 * block], "sub-range codes")
    assert_same_f32(to_host(sub_s), to_host(scales)[k0:k1], "sub-range scales")


def test_empty_and_rejected_calls():
    dx = torch.zeros(512, dtype=torch.bfloat16, device="cuda:0")
    c, s = qar.qar_quantize_blocks(dx[:0], 256)             # n == 0: nothing enqueued
    assert c.numel() == 0
    with pytest.raises(qar.QarError):
        qar.qar_quantize_blocks(dx[:300], 100)
    with pytest.raises(qar.QarError):
        qar.qar_quantize_blocks(dx[1:257], 256)             # 2-byte offset: misaligned
    codes = torch.zeros(512, dtype=torch.int8, device="cuda:0")
    scales = torch.zeros(2, dtype=torch.float32, device="cuda:0")
    with pytest.raises(qar.QarError):
        qar.qar_reduce_quantized([codes] * 33, [scales] * 33, 256)
    torch.cuda.synchronize()


def test_golden_cases_on_gpu():
    g = gc.load()
    B = g["block"]
    for case in g["quantize"]:
        x = gc.pad(case["x"], B)
        for xin in (torch.from_numpy(x).cuda(), torch.from_numpy(x).cuda().to(torch.bfloat16)):
            codes, scales = qar.qar_quantize_blocks(xin, B)
            k = len(case["codes"])
            assert list(to_host(codes)[:k]) == case["codes"], case["name"]
            want_s = gc.bits_to_f32(case["scale_bits"]) if "scale_bits" in case else np.float32(case["scale"])
            assert f32_bits(to_host(scales))[0] == f32_bits(want_s)[()], case["name"]
            y = to_host(qar.qar_dequantize(codes, scales, B, out_dtype=torch.float32))
            if "dequant" in case:
                assert np.array_equal(y[:k], np.float32(case["dequant"])), case["name"]
            for i, h in enumerate(case.get("dequant_bits", [])):
                if h is not None:
                    assert f32_bits(y)[i] == int(h, 16), (case["name"], i)
    for case in g["reduce"]:
        qs = [qar.qar_quantize_blocks(torch.from_numpy(gc.pad(r, B)).cuda(), B) for r in case["ranks"]]
        oc, os_ = qar.qar_reduce_quantized([q[0] for q in qs], [q[1] for q in qs], B)
        assert to_host(os_)[0] == np.float32(case["scale"]), case["name"]
        assert list(to_host(oc)[:len(case["codes"])]) == case["codes"], case["name"]
    for case in g["ring_step"]:
        codes = torch.from_numpy(gc.pad(case["codes_in"], B, np.int8)).cuda()
        scales = torch.tensor([case["scale_in"]], dtype=torch.float32, device="cuda:0")
        local = torch.from_numpy(gc.pad(case["local"], B)).cuda().to(torch.bfloat16)
        oc, os_ = qar.qar_ring_step(codes, scales, local, B)
        assert to_host(os_)[0] == np.float32(case["scale"]), case["name"]
        assert list(to_host(oc)[:len(case["codes"])]) == case["codes"], case["name"]


def test_beyond_2_pow_31_elements(oracle_lib):
    """n above 2**31 (64-bit element offsets): quantize and dequantize bf16,
    checked against the oracle on sampled blocks and the last blocks."""
    block = 256
    n = (1 << 31) + 3 * TILE + 7 * block
    say(f"large n={n}")
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(123)
    x.normal_(0.0, 1.0, generator=g)
    codes, scales = qar.qar_quantize_blocks(x, block)
    y = qar.qar_dequantize(codes, scales, block, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    nb = n // block
    rng = np.random.default_rng(5)
    picks = np.concatenate([rng.choice(nb, 2000, replace=False), np.arange(nb - 40, nb)])
    idx = torch.from_numpy((picks[:, None] * block + np.arange(block)).reshape(-1)).cuda()
    xs = to_host(x[idx])
    wc, ws = oracle_lib.quantize(xs, block)
    assert_same_codes(to_host(codes[idx]), wc, "codes")
    assert_same_f32(to_host(scales[torch.from_numpy(picks).cuda()]), ws, "scales")
    assert_same_bits16(to_host(y[idx]), oracle_lib.dequantize(wc, ws, block, "bf16"), "dequantized")
    del x, codes, scales, y
    torch.cuda.empty_cache()


def test_reduce_beyond_2_pow_31_elements(oracle_lib):
    """The one-kernel step and the plain reduce with N = 2 at n above 2**31,
    checked against the oracle on sampled blocks and the last blocks."""
    block = 128
    n = (1 << 31) + 5 * TILE + 3 * block
    say(f"large reduce n={n}")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(321)
    x0 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 1.0, generator=g)
    x1 = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 3.0, generator=g)
    c1, s1 = qar.qar_quantize_blocks(x1, block)
    c0 = torch.empty(n, dtype=torch.int8, device="cuda:0")
    s0 = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    fc, fs = qar.qar_quantize_reduce(x0, 0, [c0, c1], [s0, s1], block, out=out)
    rc, rs = qar.qar_reduce_quantized([c0, c1], [s0, s1], block)
    torch.cuda.synchronize()
    nb = n // block
    rng = np.random.default_rng(6)
    picks = np.concatenate([rng.choice(nb, 2000, replace=False), np.arange(nb - 40, nb)])
    pk = torch.from_numpy(picks).cuda()
    idx = torch.from_numpy((picks[:, None] * block + np.arange(block)).reshape(-1)).cuda()
    q = [oracle_lib.quantize(to_host(x[idx]), block) for x in (x0, x1)]
    wc, ws = oracle_lib.reduce([a for a, _ in q], [b for _, b in q], block)
    assert_same_codes(to_host(c0[idx]), q[0][0], "own codes")
    for c, s, what in ((fc, fs, "one-kernel step"), (rc, rs, "reduce")):
        assert_same_codes(to_host(c[idx]), wc, f"{what} codes")
        assert_same_f32(to_host(s[pk]), ws, f"{what} scales")
    assert_same_bits16(to_host(out[idx]), oracle_lib.dequantize(wc, ws, block, "bf16"), "out")
    del x0, x1, c0, c1, s0, s1, out, fc, fs, rc, rs
    torch.cuda.empty_cache()
