"""Host <-> device helpers for the GPU tests (numpy arrays as produced by the
generator and the oracle; bf16 travels as uint16 bit patterns)."""
import numpy as np
import torch

from block_wise_int8_amd import synth

TILE = 4096
SUM_OUTLIER = 9.0e36     # 32 of them still sum below the largest binary32


def ragged_n(block: int, tiles: int = 3) -> int:
    """Several 4096-element tiles plus a tail of 5 blocks."""
    return tiles * TILE + 5 * block


def mixed_f32(seed: int, n: int, block: int, outlier: float = 3.0e38) -> np.ndarray:
    """fp32 data with per-block magnitudes across the range plus special
    blocks: all zero, signed zeros, constant, subnormal, one outlier.  Data
    that is summed takes a smaller outlier so that no binary32 sum
    overflows (the method is undefined for an infinite sum)."""
    x = synth.wide_range_f32(seed, n, block, log2_span=50)
    nb = n // block
    rng = np.random.default_rng(seed + 1)
    b = rng.permutation(nb)[:6] * block
    x[b[0]:b[0] + block] = 0.0
    x[b[1]:b[1] + block] = -0.0
    x[b[1] + 3] = 1.0
    x[b[2]:b[2] + block] = np.float32(-3.25)
    x[b[3]:b[3] + block] = (rng.normal(0, 1, block) * 2.0 ** -140).astype(np.float32)
    x[b[4]:b[4] + block] = (rng.normal(0, 1, block) * 2.0 ** -149).astype(np.float32)
    x[b[5] + 7] = np.float32(outlier)
    return x


def mixed_bf16(seed: int, n: int, block: int, outlier: float = 3.0e38) -> np.ndarray:
    return synth.f32_to_bf16_bits(mixed_f32(seed, n, block, outlier))


def to_dev(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def assert_same_codes(got: np.ndarray, want: np.ndarray, what: str) -> None:
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {want.size} codes differ; first at {bad[:5]}: "
                           f"got {got[bad[:5]]}, want {want[bad[:5]]}")


def assert_same_f32(got: np.ndarray, want: np.ndarray, what: str) -> None:
    g, w = f32_bits(got), f32_bits(want)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {w.size} values differ; first at {bad[:5]}: "
                           f"got {np.asarray(got)[bad[:5]]}, want {np.asarray(want)[bad[:5]]}")


def assert_same_bits16(got: np.ndarray, want: np.ndarray, what: str) -> None:
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {want.size} bf16 values differ; first at {bad[:5]}: "
                           f"got {got[bad[:5]]}, want {want[bad[:5]]}")


def say(*a) -> None:
    print(*a, flush=True)


def oracle_allreduce(o, xs, block, schedule, nchunks):
    """The simulated AllReduce composed from oracle calls: one-shot (quantize
    every rank, reduce, dequantize) or ring by chunks (chunk c of
    ceil(nb / nchunks) blocks starts at rank c mod N).  Returns the result's
    codes, scales and dequantized values."""
    n = xs[0].size
    kind = "bf16" if xs[0].dtype == np.uint16 else "f32"
    if schedule == "one_shot":
        qs = [o.quantize(x, block) for x in xs]
        c, s = o.reduce([q[0] for q in qs], [q[1] for q in qs], block)
        return c, s, o.dequantize(c, s, block, kind)
    nb = n // block
    chunks = min(nchunks, nb)
    per = -(-nb // chunks)
    codes = np.empty(n, np.int8)
    scales = np.empty(nb, np.float32)
    out = np.empty(n, xs[0].dtype)
    N = len(xs)
    for ch in range(chunks):
        b0 = ch * per
        if b0 >= nb:
            break
        b1 = min(nb, b0 + per)
        sl = slice(b0 * block, b1 * block)
        s0 = ch % N
        c, s = o.quantize(xs[s0][sl], block)
        for k in range(1, N):
            c, s = o.ring_step(c, s, xs[(s0 + k) % N][sl], block)
        codes[sl], scales[b0:b1], out[sl] = c, s, o.dequantize(c, s, block, kind)
    return codes, scales, out
