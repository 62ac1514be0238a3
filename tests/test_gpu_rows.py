"""Row-bounded blocks ([rows, row_len], the block grid restarting at each
row) through the C ABI, against the oracle applied row by row (the oracle
quantizes any block length and a partial last block).  Bit-exact."""
import os

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth
from gpu_util import assert_same_bits16, assert_same_codes, assert_same_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# (rows, row_len, block): partial last blocks of 64, 128, 36, 8 and 37
# elements, a row shorter than one block, and a shape on the flat path
SHAPES = [(17, 2880, 256), (9, 1152, 256), (33, 100, 64), (5, 5000, 128), (40, 37, 64), (6, 5376, 256)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _data(seed, rows, row_len, kind, outlier=3.0e38):
    rng = np.random.default_rng(seed)
    v = rng.normal(0, 1, (rows, row_len)) * np.exp(rng.normal(0, 6, (rows, 1)))
    v[rng.integers(0, rows), rng.integers(0, row_len)] = outlier
    v[min(1, rows - 1), :] = 0.0                                      # an all-zero row
    v = v.astype(np.float32)
    return synth.f32_to_bf16_bits(v).reshape(rows, row_len) if kind == "bf16" else v


def _dev2(a, rows, row_len):
    return to_dev(a.reshape(-1)).view(rows, row_len)


def _oracle_quantize_rows(o, x, block):
    parts = [o.quantize(row, block) for row in x]
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _split(codes, scales, rows, row_len, block):
    per = -(-row_len // block)
    return codes.reshape(rows, row_len), scales.reshape(rows, per)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("rows,row_len,block", SHAPES)
def test_quantize_and_dequantize_rows(oracle_lib, rows, row_len, block, kind):
    x = _data(rows * 7 + row_len, rows, row_len, kind)
    say(f"rows quantize {rows}x{row_len} B={block} {kind}")
    codes, scales = qar.qar_quantize_rows(_dev2(x, rows, row_len), block)
    y = qar.qar_dequantize_rows(codes, scales, rows, row_len, block,
                                out_dtype=torch.bfloat16 if kind == "bf16" else torch.float32)
    torch.cuda.synchronize()
    wc, ws = _oracle_quantize_rows(oracle_lib, x, block)
    assert_same_codes(to_host(codes), wc, "codes")
    assert_same_f32(to_host(scales), ws, "scales")
    c2, s2 = _split(wc, ws, rows, row_len, block)
    want = np.concatenate([oracle_lib.dequantize(c2[r], s2[r], block, kind) for r in range(rows)])
    if kind == "bf16":
        assert_same_bits16(to_host(y).reshape(-1), want, "dequantized")
    else:
        assert_same_f32(to_host(y).reshape(-1), want, "dequantized")


@pytest.mark.parametrize("out", [None, "bf16", "f32"])
@pytest.mark.parametrize("nranks", [1, 2, 3, 8, 12])
@pytest.mark.parametrize("rows,row_len,block", SHAPES[:4])
def test_reduce_rows(oracle_lib, rows, row_len, block, nranks, out):
    xs = [_data(100 * r + row_len, rows, row_len, "bf16", outlier=9.0e36) for r in range(nranks)]
    say(f"rows reduce N={nranks} {rows}x{row_len} B={block} out={out}")
    qs = [qar.qar_quantize_rows(_dev2(x, rows, row_len), block) for x in xs]
    o = None if out is None else torch.empty(rows * row_len, device="cuda:0",
                                             dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    oc, os_ = qar.qar_reduce_quantized_rows([q[0] for q in qs], [q[1] for q in qs], rows, row_len, block, out=o)
    torch.cuda.synchronize()
    per_rank = [_split(*_oracle_quantize_rows(oracle_lib, x, block), rows, row_len, block) for x in xs]
    wc, ws = [], []
    for r in range(rows):
        c, s = oracle_lib.reduce([p[0][r] for p in per_rank], [p[1][r] for p in per_rank], block)
        wc.append(c), ws.append(s)
    wc, ws = np.concatenate(wc), np.concatenate(ws)
    assert_same_codes(to_host(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    if out is not None:
        c2, s2 = _split(wc, ws, rows, row_len, block)
        want = np.concatenate([oracle_lib.dequantize(c2[r], s2[r], block, out) for r in range(rows)])
        if out == "bf16":
            assert_same_bits16(to_host(o), want, "fused out")
        else:
            assert_same_f32(to_host(o), want, "fused out")


def test_rows_reduce_at_bench_shape(oracle_lib):
    """The row-bounded reduce at the shape bench.py times, N = 8 x [8192,
    2880] bf16, B = 256 (every row ends in a partial block of 64): no output
    (16 elements per lane), bf16 and fp32 output (8 per lane), each against
    the oracle row by row."""
    rows, row_len, B, N = 8192, 2880, 256, 8
    xs = [_data(500 + r, rows, row_len, "bf16", outlier=9.0e36) for r in range(N)]
    per_rank = [_split(*_oracle_quantize_rows(oracle_lib, x, B), rows, row_len, B) for x in xs]
    del xs
    dc = [to_dev(p[0].reshape(-1)) for p in per_rank]
    ds = [to_dev(p[1].reshape(-1)) for p in per_rank]
    red = [oracle_lib.reduce([p[0][r] for p in per_rank], [p[1][r] for p in per_rank], B) for r in range(rows)]
    wc, ws = np.concatenate([c for c, _ in red]), np.concatenate([s for _, s in red])
    for out in (None, "bf16", "f32"):
        say(f"rows reduce at the bench shape N={N} {rows}x{row_len} B={B} out={out}")
        o = None if out is None else torch.empty(rows * row_len, device="cuda:0",
                                                 dtype=torch.bfloat16 if out == "bf16" else torch.float32)
        oc, os_ = qar.qar_reduce_quantized_rows(dc, ds, rows, row_len, B, out=o)
        torch.cuda.synchronize()
        assert_same_codes(to_host(oc), wc, f"codes (out={out})")
        assert_same_f32(to_host(os_), ws, f"scales (out={out})")
        if out is not None:
            want = np.concatenate([oracle_lib.dequantize(c, s, B, out) for c, s in red])
            if out == "bf16":
                assert_same_bits16(to_host(o), want, "fused out")
            else:
                assert_same_f32(to_host(o), want, "fused out")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("rows,row_len,block", SHAPES[:5])
def test_ring_step_rows(oracle_lib, rows, row_len, block, kind, in_place):
    x0 = _data(5 + row_len, rows, row_len, kind, outlier=9.0e36)
    x1 = _data(6 + row_len, rows, row_len, kind, outlier=9.0e36)
    say(f"rows ring {rows}x{row_len} B={block} {kind} in_place={in_place}")
    c, s = qar.qar_quantize_rows(_dev2(x0, rows, row_len), block)
    if in_place:
        oc, os_ = qar.qar_ring_step_rows(c, s, _dev2(x1, rows, row_len), block, codes_out=c, scales_out=s)
    else:
        oc, os_ = qar.qar_ring_step_rows(c, s, _dev2(x1, rows, row_len), block)
    torch.cuda.synchronize()
    c0, s0 = _split(*_oracle_quantize_rows(oracle_lib, x0, block), rows, row_len, block)
    parts = [oracle_lib.ring_step(c0[r], s0[r], x1[r], block) for r in range(rows)]
    assert_same_codes(to_host(oc), np.concatenate([p[0] for p in parts]), "codes")
    assert_same_f32(to_host(os_), np.concatenate([p[1] for p in parts]), "scales")


def test_rows_on_the_flat_path_equal_flat_calls():
    rows, row_len, block = 6, 5376, 256
    x = to_dev(_data(3, rows, row_len, "bf16").reshape(-1))
    c1, s1 = qar.qar_quantize_rows(x.view(rows, row_len), block)
    c2, s2 = qar.qar_quantize_blocks(x, block)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_rows_unaligned_pointers_take_the_general_path(oracle_lib):
    """row_len % 16 == 0 but the data starts 2 bytes into an allocation:
    the element-wise kernels run, with the same results."""
    rows, row_len, block = 7, 2880, 256
    x = _data(99, rows, row_len, "bf16")
    base = torch.empty(rows * row_len + 8, dtype=torch.bfloat16, device="cuda:0")
    view = base[1:1 + rows * row_len]
    view.copy_(to_dev(x.reshape(-1)))
    codes = torch.empty(rows * row_len + 16, dtype=torch.int8, device="cuda:0")[3:3 + rows * row_len]
    c, s = qar.qar_quantize_rows(view.view(rows, row_len), block, codes=codes)
    torch.cuda.synchronize()
    wc, ws = _oracle_quantize_rows(oracle_lib, x, block)
    assert_same_codes(to_host(c), wc, "codes")
    assert_same_f32(to_host(s), ws, "scales")


EDGE_SHAPES = [(1, 16, 64), (3, 1, 64), (2, 17, 256), (1, 4096 + 16, 256), (4, 64, 64), (2, 255, 256)]


@pytest.mark.parametrize("rows,row_len,block", EDGE_SHAPES)
def test_rows_edge_shapes(oracle_lib, rows, row_len, block):
    """Edge shapes: one-element rows, one row of a single lane group, one row
    just past a tile, rows of exactly one block and one element short of a
    block -- quantize, dequantize, the reduce (N = 3, bf16 out) and a ring
    step, row by row against the oracle."""
    rng = np.random.default_rng(rows * 1000 + row_len)
    xs = [synth.f32_to_bf16_bits((rng.normal(0, 1, (rows, row_len)) * np.exp(rng.normal(0, 4, (rows, 1))))
                                 .astype(np.float32)).reshape(rows, row_len) for _ in range(3)]
    say(f"rows edge {rows}x{row_len} B={block}")
    qs = [qar.qar_quantize_rows(_dev2(x, rows, row_len), block) for x in xs]
    y = qar.qar_dequantize_rows(qs[0][0], qs[0][1], rows, row_len, block, out_dtype=torch.bfloat16)
    o = torch.empty(rows * row_len, device="cuda:0", dtype=torch.bfloat16)
    oc, os_ = qar.qar_reduce_quantized_rows([q[0] for q in qs], [q[1] for q in qs], rows, row_len, block, out=o)
    gc_, gs_ = qar.qar_ring_step_rows(qs[0][0], qs[0][1], _dev2(xs[1], rows, row_len), block)
    torch.cuda.synchronize()
    per_rank = [_split(*_oracle_quantize_rows(oracle_lib, x, block), rows, row_len, block) for x in xs]
    for r, (q, p) in enumerate(zip(qs, per_rank)):
        assert_same_codes(to_host(q[0]), p[0].reshape(-1), f"rank {r} codes")
        assert_same_f32(to_host(q[1]), p[1].reshape(-1), f"rank {r} scales")
    want_y = np.concatenate([oracle_lib.dequantize(per_rank[0][0][r], per_rank[0][1][r], block, "bf16")
                             for r in range(rows)])
    assert_same_bits16(to_host(y).reshape(-1), want_y, "dequantized")
    red = [oracle_lib.reduce([p[0][r] for p in per_rank], [p[1][r] for p in per_rank], block) for r in range(rows)]
    assert_same_codes(to_host(oc), np.concatenate([c for c, _ in red]), "reduce codes")
    assert_same_f32(to_host(os_), np.concatenate([s for _, s in red]), "reduce scales")
    assert_same_bits16(to_host(o), np.concatenate([oracle_lib.dequantize(c, s, block, "bf16") for c, s in red]),
                       "reduce out")
    ring = [oracle_lib.ring_step(per_rank[0][0][r], per_rank[0][1][r], xs[1][r], block) for r in range(rows)]
    assert_same_codes(to_host(gc_), np.concatenate([c for c, _ in ring]), "ring codes")
    assert_same_f32(to_host(gs_), np.concatenate([s for _, s in ring]), "ring scales")


RANDOM_ROW_CASES = int(os.environ.get("QAR_RANDOM_CASES", "200")) // 4


@pytest.mark.parametrize("case", range(RANDOM_ROW_CASES))
def test_rows_random_configuration(oracle_lib, case):
    """Seeded random row shapes (row lengths with and without a partial last
    block, on and off the 16-element lane grid), block size, rank count,
    input and output types, through every row call against the oracle row by
    row."""
    rng = np.random.default_rng(30_000 + case)
    block = int(rng.choice([64, 128, 256]))
    rows = int(rng.integers(1, 24))
    row_len = int(rng.integers(1, 3 * block + 1)) * (16 if rng.random() < 0.5 else 1)
    nranks = int(rng.integers(1, 10))
    kind = str(rng.choice(["bf16", "f32"]))
    out_kind = str(rng.choice(["none", "bf16", "f32"]))
    say(f"rows random case {case}: {rows}x{row_len} B={block} N={nranks} {kind} out={out_kind}")
    xs = []
    for _ in range(nranks):
        v = (rng.normal(0, 1, (rows, row_len)) * np.exp(rng.normal(0, 4, (rows, 1)))).astype(np.float32)
        xs.append(synth.f32_to_bf16_bits(v).reshape(rows, row_len) if kind == "bf16" else v)
    qs = [qar.qar_quantize_rows(_dev2(x, rows, row_len), block) for x in xs]
    o = None if out_kind == "none" else torch.empty(rows * row_len, device="cuda:0",
                                                    dtype=torch.bfloat16 if out_kind == "bf16" else torch.float32)
    oc, os_ = qar.qar_reduce_quantized_rows([q[0] for q in qs], [q[1] for q in qs], rows, row_len, block, out=o)
    gc_, gs_ = qar.qar_ring_step_rows(qs[0][0], qs[0][1], _dev2(xs[-1], rows, row_len), block)
    y = qar.qar_dequantize_rows(oc, os_, rows, row_len, block,
                                out_dtype=torch.bfloat16 if kind == "bf16" else torch.float32)
    torch.cuda.synchronize()
    per_rank = [_split(*_oracle_quantize_rows(oracle_lib, x, block), rows, row_len, block) for x in xs]
    for r, (q, p) in enumerate(zip(qs, per_rank)):
        assert_same_codes(to_host(q[0]), p[0].reshape(-1), f"rank {r} codes")
        assert_same_f32(to_host(q[1]), p[1].reshape(-1), f"rank {r} scales")
    red = [oracle_lib.reduce([p[0][r] for p in per_rank], [p[1][r] for p in per_rank], block) for r in range(rows)]
    wc, ws = np.concatenate([c for c, _ in red]), np.concatenate([s for _, s in red])
    assert_same_codes(to_host(oc), wc, "reduce codes")
    assert_same_f32(to_host(os_), ws, "reduce scales")
    if o is not None:
        want = np.concatenate([oracle_lib.dequantize(c, s, block, out_kind) for c, s in red])
        if out_kind == "bf16":
            assert_same_bits16(to_host(o), want, "fused out")
        else:
            assert_same_f32(to_host(o), want, "fused out")
    want_y = np.concatenate([oracle_lib.dequantize(c, s, block, kind) for c, s in red])
    if kind == "bf16":
        assert_same_bits16(to_host(y).reshape(-1), want_y, "dequantized")
    else:
        assert_same_f32(to_host(y).reshape(-1), want_y, "dequantized")
    ring = [oracle_lib.ring_step(per_rank[0][0][r], per_rank[0][1][r], xs[-1][r], block) for r in range(rows)]
    assert_same_codes(to_host(gc_), np.concatenate([c for c, _ in ring]), "ring codes")
    assert_same_f32(to_host(gs_), np.concatenate([s for _, s in ring]), "ring scales")
