"""Several host threads calling libqar at once, each on its own streams: the
library keeps no shared mutable state (the pipelined call's events are per
thread and device), so every thread's results must equal the oracle's."""
import threading

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar
from gpu_util import SUM_OUTLIER, assert_same_bits16, assert_same_codes, assert_same_f32, mixed_bf16, ragged_n, \
    say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()
    torch.cuda.init()


def test_concurrent_host_threads(oracle_lib):
    T, N, block, iters = 4, 4, 128, 5
    n = ragged_n(block)
    xs = [[mixed_bf16(7000 + 10 * t + r, n, block, SUM_OUTLIER) for r in range(N)] for t in range(T)]
    want = []
    for t in range(T):
        q = [oracle_lib.quantize(x, block) for x in xs[t]]
        wc, ws = oracle_lib.reduce([c for c, _ in q], [s for _, s in q], block)
        want.append((q, wc, ws, oracle_lib.dequantize(wc, ws, block, "bf16")))

    results, errors = [None] * T, []

    def work(t):
        try:
            main, side = torch.cuda.Stream(), [torch.cuda.Stream(), torch.cuda.Stream()]
            with torch.cuda.stream(main):
                x = [to_dev(a) for a in xs[t]]
                codes = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(N)]
                scales = [torch.empty(n // block, dtype=torch.float32, device="cuda:0") for _ in range(N)]
                outs = {k: (torch.empty(n, dtype=torch.int8, device="cuda:0"),
                            torch.empty(n // block, dtype=torch.float32, device="cuda:0"),
                            torch.empty(n, dtype=torch.bfloat16, device="cuda:0"))
                        for k in ("reduce", "pipelined", "step")}
                got = []
                for it in range(iters):
                    for r in range(N):
                        qar.qar_quantize_blocks(x[r], block, codes[r], scales[r])
                    c, s, o = outs["reduce"]
                    qar.qar_reduce_quantized(codes, scales, block, c, s, out=o)
                    c, s, o = outs["pipelined"]
                    qar.qar_reduce_quantized_pipelined(codes, scales, block, 4, side, c, s, out=o)
                    own = it % N
                    c, s, o = outs["step"]
                    qar.qar_quantize_reduce(x[own], own, codes, scales, block, c, s, out=o)
                    main.synchronize()
                    got.append({k: tuple(to_host(a) for a in v) for k, v in outs.items()}
                               | {"codes": [to_host(a) for a in codes], "scales": [to_host(a) for a in scales]})
            results[t] = got
        except Exception as e:  # reported by the main thread
            errors.append((t, repr(e)))

    say(f"{T} host threads x {iters} iterations, N={N}, n={n}")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(T)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a host thread did not finish"
    assert not errors, errors
    for t in range(T):
        q, wc, ws, wy = want[t]
        for it, got in enumerate(results[t]):
            what = f"thread {t} iteration {it}"
            for r in range(N):
                assert_same_codes(got["codes"][r], q[r][0], f"{what} rank {r} codes")
                assert_same_f32(got["scales"][r], q[r][1], f"{what} rank {r} scales")
            for k in ("reduce", "pipelined", "step"):
                c, s, o = got[k]
                assert_same_codes(c, wc, f"{what} {k} codes")
                assert_same_f32(s, ws, f"{what} {k} scales")
                assert_same_bits16(o, wy, f"{what} {k} bf16 out")
