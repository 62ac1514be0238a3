"""qar_allreduce_simulated_static, the entry point for callers that cannot
allocate, against qar_allreduce_simulated (caller workspaces, same schedule
and chunking): bit-identical results, called through the C ABI, two calls
in a row with the second one smaller (the static workspace keeps the first
call's bytes; nothing the second reads may come from them)."""
import ctypes

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ranks(seed, nranks, n, dtype):
    if dtype == "bf16":
        hs = synth.uniform_bf16(seed, nranks, n)
        return [torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16) for h in hs]
    return [torch.from_numpy(h).to(DEV) for h in synth.uniform_f32(seed, nranks, n)]


def _static_via_abi(xs, block, schedule, nchunks, out):
    """The C entry point called directly through ctypes."""
    L = qar.lib()
    xp = (ctypes.c_void_p * len(xs))(*[x.data_ptr() for x in xs])
    sched = qar.QAR_SCHEDULE_ONE_SHOT if schedule == "one_shot" else qar.QAR_SCHEDULE_RING
    return L.qar_allreduce_simulated_static(ctypes.cast(xp, ctypes.c_void_p), qar._dtype_code(xs[0].dtype),
                                            len(xs), xs[0].numel(), block, sched, out.data_ptr(), nchunks,
                                            torch.cuda.current_stream().cuda_stream)


# (nranks, n, block, nchunks): the first call of each pair is the larger one
PAIRS = [
    ((4, 1 << 21, 256, 4), (3, 64 * 1000, 64, 2)),
    ((8, 1 << 20, 128, 3), (2, 4096, 128, 1)),
]


@pytest.mark.parametrize("schedule", ["one_shot", "ring"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_static_equals_workspace_call_twice_in_a_row(schedule, dtype, pair):
    for k, (N, n, B, nchunks) in enumerate(PAIRS[pair]):
        print(f"static allreduce: {schedule} {dtype} N={N} n={n} B={B} chunks={nchunks}", flush=True)
        xs = _ranks(100 * pair + k, N, n, dtype)
        ref = qar.qar_allreduce_simulated(xs, B, schedule, nchunks, [torch.cuda.current_stream()])
        got = torch.full_like(ref, float("nan"))
        assert _static_via_abi(xs, B, schedule, nchunks, got) == qar.QAR_OK
        torch.cuda.synchronize()
        iv = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(got.view(iv), ref.view(iv)), (schedule, dtype, N, n, B, nchunks)


def test_static_binding_and_capacity():
    xs = _ranks(7, 4, 1 << 16, "bf16")
    ref = qar.qar_allreduce_simulated(xs, 256, "one_shot", 2, [torch.cuda.current_stream()])
    got = qar.qar_allreduce_simulated_static(xs, 256, "one_shot", 2)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # one-shot over 8 ranks of 2^23 elements stages 8 x 8.4 MB > 64 MiB: refused, nothing enqueued
    big = [torch.empty(1 << 23, dtype=torch.bfloat16, device=DEV)] * 8
    with pytest.raises(qar.QarError, match="static workspace"):
        qar.qar_allreduce_simulated_static(big, 256, "one_shot")
    torch.cuda.synchronize()
