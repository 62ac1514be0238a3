"""libqar inside HIP graphs.  The library never allocates, frees or
synchronizes, and its multi-stream calls fork and join their side streams
with events, so a caller can capture them (here with torch.cuda.graph) and
replay the graph.  Each replay runs on new inputs copied in eagerly between
replays, and its outputs must equal, bit for bit, an eager call on the same
inputs (and, for the first replay, the oracle)."""
import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar
from gpu_util import (SUM_OUTLIER, assert_same_bits16, assert_same_codes, assert_same_f32, mixed_bf16, ragged_n,
                      say, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _same(a: torch.Tensor, b: torch.Tensor, what: str) -> None:
    x = a.contiguous().view(torch.uint8).cpu().numpy()
    y = b.contiguous().view(torch.uint8).cpu().numpy()
    bad = np.nonzero(x != y)[0]
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[:5]}"


def test_pipelined_reduce_replays(oracle_lib):
    block, nranks, nchunks = 256, 4, 16
    n = ragged_n(block, tiles=8)
    streams = [torch.cuda.Stream() for _ in range(4)]
    dc = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(nranks)]
    ds = [torch.empty(n // block, dtype=torch.float32, device="cuda:0") for _ in range(nranks)]
    co = torch.empty(n, dtype=torch.int8, device="cuda:0")
    so = torch.empty(n // block, dtype=torch.float32, device="cuda:0")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")

    def load_inputs(seed):
        xs = [mixed_bf16(seed + r, n, block, SUM_OUTLIER) for r in range(nranks)]
        qs = [oracle_lib.quantize(x, block) for x in xs]
        for r, (c, s) in enumerate(qs):
            dc[r].copy_(to_dev(c))
            ds[r].copy_(to_dev(s))
        return qs

    load_inputs(1000)
    qar.qar_reduce_quantized_pipelined(dc, ds, block, nchunks, streams, co, so, out=out)   # events made eagerly
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qar.qar_reduce_quantized_pipelined(dc, ds, block, nchunks, streams, co, so, out=out)
    for rep in range(3):
        qs = load_inputs(1100 + 10 * rep)
        torch.cuda.synchronize()
        say(f"graph replay {rep}: pipelined reduce, {nchunks} chunks on 4 streams")
        g.replay()
        torch.cuda.synchronize()
        ec, es, eo = torch.empty_like(co), torch.empty_like(so), torch.empty_like(out)
        qar.qar_reduce_quantized_pipelined(dc, ds, block, nchunks, streams, ec, es, out=eo)
        torch.cuda.synchronize()
        _same(co, ec, f"replay {rep} codes")
        _same(so, es, f"replay {rep} scales")
        _same(out, eo, f"replay {rep} out")
        if rep == 0:
            wc, ws = oracle_lib.reduce([q[0] for q in qs], [q[1] for q in qs], block)
            assert_same_codes(to_host(co), wc, "replay codes vs oracle")
            assert_same_f32(to_host(so), ws, "replay scales vs oracle")
            assert_same_bits16(to_host(out), oracle_lib.dequantize(wc, ws, block, "bf16"), "replay out vs oracle")


@pytest.mark.parametrize("schedule", ["one_shot", "ring"])
def test_allreduce_simulated_replays(oracle_lib, schedule):
    block, nranks, nchunks = 128, 4, 4
    n = ragged_n(block, tiles=6)
    streams = [torch.cuda.Stream() for _ in range(4)]
    xs = [torch.empty(n, dtype=torch.bfloat16, device="cuda:0") for _ in range(nranks)]
    nwork = nranks if schedule == "one_shot" else 1
    wc = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(nwork)]
    ws = [torch.empty(n // block, dtype=torch.float32, device="cuda:0") for _ in range(nwork)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")

    def load_inputs(seed):
        for r in range(nranks):
            xs[r].copy_(to_dev(mixed_bf16(seed + r, n, block, SUM_OUTLIER)))

    load_inputs(2000)
    qar.qar_allreduce_simulated(xs, block, schedule, nchunks, streams, out=out, workspace=(wc, ws))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qar.qar_allreduce_simulated(xs, block, schedule, nchunks, streams, out=out, workspace=(wc, ws))
    for rep in range(3):
        load_inputs(2100 + 10 * rep)
        torch.cuda.synchronize()
        say(f"graph replay {rep}: simulated all-reduce ({schedule}), {nchunks} chunks on 4 streams")
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ewc = [torch.empty_like(t) for t in wc]
        ews = [torch.empty_like(t) for t in ws]
        eo = qar.qar_allreduce_simulated(xs, block, schedule, nchunks, streams, workspace=(ewc, ews))
        torch.cuda.synchronize()
        _same(got, eo, f"{schedule} replay {rep} result")
