"""Host <-> device helpers for the GPU tests (numpy arrays as produced by the
generator and the oracle; bf16 travels as uint16 bit patterns)."""
import numpy as np
import torch


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
