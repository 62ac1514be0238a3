"""Seeded random configurations through every flat call, int8, E4M3 and
4-bit codes, against the oracle bit for bit: rank count, block size, input type,
output type, size (whole blocks, from one block to several tiles, and for
the chunked calls up to several interleaved runs) and the value distribution
all drawn per case."""
import os

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth
from gpu_util import assert_same_bits16, assert_same_codes, assert_same_f32, oracle_allreduce, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# seeds 10,000 .. 10,000 + CASES - 1; QAR_RANDOM_CASES widens the sweep
CASES = int(os.environ.get("QAR_RANDOM_CASES", "200"))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _draw(rng, n, block, dtype):
    kind = rng.integers(0, 4)
    if kind == 0:
        v = rng.normal(0, 1, n)
    elif kind == 1:
        v = rng.laplace(0, 0.5, n) * np.repeat(np.exp(rng.normal(0, 3, n // block)), block)
    elif kind == 2:
        v = rng.normal(0, 1, n)
        v[rng.integers(0, n, max(1, n // 500))] *= 1000.0
    else:
        v = rng.integers(-3, 4, n).astype(np.float64) * 0.5          # ties and zeros
    v = v.astype(np.float32)
    return synth.f32_to_bf16_bits(v) if dtype == "bf16" else v


def _same_out(got, want, dtype, what):
    if dtype == "bf16":
        assert_same_bits16(got, want, what)
    else:
        assert_same_f32(got, want, what)


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration(oracle_lib, case):
    rng = np.random.default_rng(10_000 + case)
    block = int(rng.choice([64, 128, 256]))
    # mostly one or two load groups of 8 ranks, sometimes up to the limit (four)
    nranks = int(rng.integers(1, 12)) if rng.random() < 0.8 else int(rng.integers(12, qar.QAR_MAX_RANKS + 1))
    dtype = str(rng.choice(["bf16", "f32"]))
    n = int(rng.integers(1, 3 * 4096 // block + 3)) * block
    codes_fmt = str(rng.choice(["int8", "e4m3", "int4"]))
    own = int(rng.integers(0, nranks))
    say(f"random case {case}: {codes_fmt} N={nranks} own={own} B={block} n={n} {dtype}")
    _run_case(oracle_lib, rng, block, nranks, dtype, n, codes_fmt, own)


EDGE_SIZES = {"one block": lambda b: b, "half tile minus a block": lambda b: 2048 - b, "half tile": lambda b: 2048,
              "half tile plus a block": lambda b: 2048 + b, "tile minus a block": lambda b: 4096 - b,
              "one tile": lambda b: 4096, "tile plus a block": lambda b: 4096 + b}


@pytest.mark.parametrize("nranks", [3, 6])
@pytest.mark.parametrize("size", list(EDGE_SIZES))
@pytest.mark.parametrize("block", [64, 128, 256])
@pytest.mark.parametrize("codes_fmt", ["int8", "e4m3", "int4"])
def test_edge_sizes(oracle_lib, codes_fmt, block, size, nranks):
    """Sizes at the edges of the tiling, through every flat call: a single
    block (one lane group of a wave), one block either side of and exactly a
    2,048-element tile (the kernels with 8 elements per lane, which the reduce
    takes from 6 ranks on for int8 and E4M3 codes) and a 4,096-element tile
    (16 per lane)."""
    n = EDGE_SIZES[size](block)
    rng = np.random.default_rng(20_000 + n + block + 7 * nranks)
    dtype = "bf16" if (n // block) % 2 else "f32"
    say(f"edge size: {codes_fmt} N={nranks} B={block} n={n} {dtype}")
    _run_case(oracle_lib, rng, block, nranks, dtype, n, codes_fmt, 1)


def _run_case(oracle_lib, rng, block, nranks, dtype, n, codes_fmt, own):
    if codes_fmt == "int8":
        quant, red, qred, ring, deq = (qar.qar_quantize_blocks, qar.qar_reduce_quantized, qar.qar_quantize_reduce,
                                       qar.qar_ring_step, qar.qar_dequantize)
        o_quant, o_red, o_ring, o_deq = (oracle_lib.quantize, oracle_lib.reduce, oracle_lib.ring_step,
                                         oracle_lib.dequantize)
        view = lambda t: to_host(t)
    elif codes_fmt == "int4":
        quant, red, qred, ring, deq = (qar.qar_quantize_blocks_int4, qar.qar_reduce_quantized_int4,
                                       qar.qar_quantize_reduce_int4, qar.qar_ring_step_int4, qar.qar_dequantize_int4)
        o_quant, o_ring = oracle_lib.quantize_int4, oracle_lib.ring_step_int4
        o_red = lambda c, s, b: oracle_lib.reduce_int4(c, s, b, n)
        o_deq = lambda c, s, b, k: oracle_lib.dequantize_int4(c, s, b, n, k)
        view = lambda t: to_host(t).view(np.uint8)
    else:
        quant, red, qred, ring, deq = (qar.qar_quantize_blocks_e4m3, qar.qar_reduce_quantized_e4m3,
                                       qar.qar_quantize_reduce_e4m3, qar.qar_ring_step_e4m3, qar.qar_dequantize_e4m3)
        o_quant, o_red, o_ring, o_deq = (oracle_lib.quantize_e4m3, oracle_lib.reduce_e4m3,
                                         oracle_lib.ring_step_e4m3, oracle_lib.dequantize_e4m3)
        view = lambda t: to_host(t).view(np.uint8)
    xs = [_draw(rng, n, block, dtype) for _ in range(nranks)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # quantize every rank
    q = [quant(to_dev(x), block) for x in xs]
    wq = [o_quant(x, block) for x in xs]
    # reduce with an output of the input type
    out = torch.empty(n, dtype=tdt, device="cuda:0")
    rc, rs = red([c for c, _ in q], [s for _, s in q], block, out=out)
    # the one-kernel step with rank own quantized inside
    own_c, own_s = torch.empty_like(q[own][0]), torch.empty_like(q[own][1])
    qc = [c for c, _ in q]
    qs = [s for _, s in q]
    qc[own], qs[own] = own_c, own_s
    fc, fs = qred(to_dev(xs[own]), own, qc, qs, block)
    # a ring step from rank 0 with rank N-1's data, and a dequantize
    gc_, gs_ = ring(q[0][0], q[0][1], to_dev(xs[-1]), block)
    y = deq(rc, rs, block, out_dtype=tdt)
    torch.cuda.synchronize()
    for r, ((c, s), (wc, ws)) in enumerate(zip(q, wq)):
        assert_same_codes(view(c), wc, f"rank {r} codes")
        assert_same_f32(to_host(s), ws, f"rank {r} scales")
    wc, ws = o_red([a for a, _ in wq], [b for _, b in wq], block)
    assert_same_codes(view(rc), wc, "reduce codes")
    assert_same_f32(to_host(rs), ws, "reduce scales")
    _same_out(to_host(out), o_deq(wc, ws, block, dtype), dtype, "fused out")
    _same_out(to_host(y), o_deq(wc, ws, block, dtype), dtype, "dequantize")
    assert_same_codes(view(own_c), wq[own][0], "own codes")
    assert_same_codes(view(fc), wc, "one-kernel step codes")
    assert_same_f32(to_host(fs), ws, "one-kernel step scales")
    rgc, rgs = o_ring(wq[0][0], wq[0][1], xs[-1], block)
    assert_same_codes(view(gc_), rgc, "ring codes")
    assert_same_f32(to_host(gs_), rgs, "ring scales")



@pytest.mark.parametrize("case", range(max(4, CASES // 8)))
def test_random_chunked_runs(oracle_lib, case):
    """The chunked and the pipelined reduce at sizes of zero to six runs of
    QAR_CHUNK_RUN_ELEMS plus a ragged part, with random rank, chunk and
    stream counts (the chunked call also with a fused output), so that the
    interleaved chunks' whole runs, the last partial run and chunk counts
    above the run count are all met; against the oracle."""
    rng = np.random.default_rng(50_000 + case)
    run = qar.QAR_CHUNK_RUN_ELEMS
    block = int(rng.choice([64, 128, 256]))
    nranks = int(rng.integers(1, 17))
    n = int(rng.integers(0, 7)) * run + int(rng.integers(1, run // block)) * block
    nchunks = int(rng.integers(1, 13))
    nstreams = int(rng.integers(1, 5))
    out_kind = [None, "bf16", "f32"][int(rng.integers(0, 3))]
    say(f"random chunked case {case}: N={nranks} B={block} n={n} chunks={nchunks} streams={nstreams} out={out_kind}")
    xs = [_draw(rng, n, block, "bf16") for _ in range(nranks)]
    q = [oracle_lib.quantize(x, block) for x in xs]
    dc, ds = [to_dev(c) for c, _ in q], [to_dev(s) for _, s in q]
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    out = None if out_kind is None else torch.empty(
        n, dtype=torch.bfloat16 if out_kind == "bf16" else torch.float32, device="cuda:0")
    oc = torch.empty(n, dtype=torch.int8, device="cuda:0")
    os_ = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    fork = torch.cuda.Event()                 # the chunks run after the copies above
    fork.record(cur)
    for st in streams:
        st.wait_event(fork)
    qar.qar_reduce_quantized_chunked(dc, ds, block, nchunks, streams, oc, os_, out=out)
    for st in streams:
        done = torch.cuda.Event()
        done.record(st)
        cur.wait_event(done)
    torch.cuda.synchronize()
    rc, rs = oracle_lib.reduce([c for c, _ in q], [s for _, s in q], block)
    assert_same_codes(to_host(oc), rc, "chunked codes")
    assert_same_f32(to_host(os_), rs, "chunked scales")
    if out_kind is not None:
        _same_out(to_host(out), oracle_lib.dequantize(rc, rs, block, out_kind), out_kind, "chunked out")
    # the same cut through the pipelined call, which orders the streams itself
    oc.fill_(0x55)
    os_.fill_(-1.0)
    qar.qar_reduce_quantized_pipelined(dc, ds, block, nchunks, streams, oc, os_)
    torch.cuda.synchronize()
    assert_same_codes(to_host(oc), rc, "pipelined codes")
    assert_same_f32(to_host(os_), rs, "pipelined scales")


@pytest.mark.parametrize("case", range(CASES // 4))
def test_random_pipelined_and_simulated(oracle_lib, case):
    """Seeded random chunk counts and stream counts through the pipelined
    reduce and the simulated AllReduce (one-shot and ring), against the
    oracle's reduce and its chunk-by-chunk composition."""
    rng = np.random.default_rng(40_000 + case)
    block = int(rng.choice([64, 128, 256]))
    nranks = int(rng.integers(1, 10))
    dtype = str(rng.choice(["bf16", "f32"]))
    n = int(rng.integers(1, 3 * 4096 // block + 3)) * block
    nchunks = int(rng.integers(1, 2 * (n // block) + 2))        # sometimes more chunks than blocks
    nstreams = int(rng.integers(1, 5))
    schedule = str(rng.choice(["one_shot", "ring"]))
    say(f"random pipelined case {case}: N={nranks} B={block} n={n} {dtype} chunks={nchunks} "
        f"streams={nstreams} {schedule}")
    xs = [_draw(rng, n, block, dtype) for _ in range(nranks)]
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    q = [qar.qar_quantize_blocks(to_dev(x), block) for x in xs]
    pc, ps = qar.qar_reduce_quantized_pipelined([c for c, _ in q], [s for _, s in q], block, nchunks, streams)
    nwork = nranks if schedule == "one_shot" else 1
    wc = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(nwork)]
    ws = [torch.empty(n // block, dtype=torch.float32, device="cuda:0") for _ in range(nwork)]
    out = qar.qar_allreduce_simulated([to_dev(x) for x in xs], block, schedule, nchunks, streams,
                                      workspace=(wc, ws))
    torch.cuda.synchronize()
    wq = [oracle_lib.quantize(x, block) for x in xs]
    rc, rs = oracle_lib.reduce([c for c, _ in wq], [s for _, s in wq], block)
    assert_same_codes(to_host(pc), rc, "pipelined codes")
    assert_same_f32(to_host(ps), rs, "pipelined scales")
    c, s, y = oracle_allreduce(oracle_lib, xs, block, schedule, nchunks)
    assert_same_codes(to_host(wc[0]), c, "simulated result codes")
    assert_same_f32(to_host(ws[0]), s, "simulated result scales")
    _same_out(to_host(out), y, dtype, "simulated result")
