"""ctypes binding of libqar (include/qar.h): argument marshalling only.

Every computation runs in libqar's HIP kernels; this module turns torch
tensors into device pointers, HIP streams into handles, allocates outputs
with torch when the caller passes none, and raises ``QarError`` on a
non-OK status.  A missing library raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libqar.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qar.h")

QAR_OK, QAR_ERR_INVALID_ARG, QAR_ERR_MISALIGNED, QAR_ERR_UNSUPPORTED, QAR_ERR_HIP, QAR_ERR_CAPACITY = range(6)
QAR_BF16, QAR_F32 = 0, 1
QAR_SCHEDULE_ONE_SHOT, QAR_SCHEDULE_RING = 0, 1
QAR_MAX_RANKS = 32
QAR_MAX_STREAMS = 16
QAR_STATIC_WORKSPACE_BYTES = 64 << 20
QAR_CHUNK_RUN_ELEMS = 1 << 18
BLOCK_SIZES = (64, 128, 256)

_vp, _sz, _u32, _int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int

_SIGNATURES = {
    "qar_quantize_blocks": [_vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_reduce_quantized": [_vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_quantize_reduce": [_vp, _int, _u32, _vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_reduce_quantized_pipelined": [_vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _u32, _vp, _u32, _vp],
    "qar_reduce_quantized_chunked": [_vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _u32, _vp, _u32],
    "qar_ring_step": [_vp, _vp, _vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_dequantize": [_vp, _vp, _sz, _u32, _vp, _int, _vp],
    "qar_reduce_unquantized": [_vp, _u32, _sz, _int, _vp, _vp],
    "qar_quantize_rows": [_vp, _int, _sz, _sz, _u32, _vp, _vp, _vp],
    "qar_reduce_quantized_rows": [_vp, _vp, _u32, _sz, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_ring_step_rows": [_vp, _vp, _vp, _int, _sz, _sz, _u32, _vp, _vp, _vp],
    "qar_dequantize_rows": [_vp, _vp, _sz, _sz, _u32, _vp, _int, _vp],
    "qar_allreduce_simulated": [_vp, _int, _u32, _sz, _u32, _int, _vp, _vp, _vp, _u32, _vp, _u32, _vp],
    "qar_allreduce_simulated_static": [_vp, _int, _u32, _sz, _u32, _int, _vp, _u32, _vp],
    "qar_quantize_blocks_e4m3": [_vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_reduce_quantized_e4m3": [_vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_quantize_reduce_e4m3": [_vp, _int, _u32, _vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_ring_step_e4m3": [_vp, _vp, _vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_dequantize_e4m3": [_vp, _vp, _sz, _u32, _vp, _int, _vp],
    "qar_quantize_blocks_int4": [_vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_reduce_quantized_int4": [_vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_quantize_reduce_int4": [_vp, _int, _u32, _vp, _vp, _u32, _sz, _u32, _vp, _vp, _vp, _int, _vp],
    "qar_ring_step_int4": [_vp, _vp, _vp, _int, _sz, _u32, _vp, _vp, _vp],
    "qar_dequantize_int4": [_vp, _vp, _sz, _u32, _vp, _int, _vp],
    "qar_status_string": [_int],
    "qar_last_error": [],
}


class QarError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        L = lib()
        text = L.qar_status_string(status).decode()
        detail = L.qar_last_error().decode() if status in (QAR_ERR_HIP, QAR_ERR_CAPACITY) else ""
        super().__init__(f"{where}: {text}" + (f" ({detail})" if detail else ""))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqar (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"libqar is not built: {LIBRARY} is missing "
                               "(build it with __graft_entry__.build() or block_wise_int8_amd/build.py)")
        L = ctypes.CDLL(LIBRARY)
        for name, args in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name in ("qar_status_string", "qar_last_error") else _int
        _lib = L
    return _lib


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/qar.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qar_\w+)\s*\(", text, re.M)))


# ----------------------------------------------------------------------------
# marshalling helpers


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return QAR_BF16
    if dt == torch.float32:
        return QAR_F32
    raise TypeError(f"libqar handles bfloat16 and float32 data, not {dt}")


def _dev(t: torch.Tensor, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _check(status: int, where: str) -> None:
    if status != QAR_OK:
        raise QarError(status, where)


def _ptrs(ts: list[torch.Tensor]):
    arr = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    return arr


# The C ABI sees only pointers, so a tensor too small for the call would be
# read or written past its end.  Every tensor handed to the library is
# therefore checked here first: type, element count and device.
_CODE_DTYPES = (torch.int8, torch.uint8)     # any byte container holds codes
_DATA_DTYPES = (torch.bfloat16, torch.float32)


def _expect(t: torch.Tensor, what: str, numel: int, dtypes: tuple, device: torch.device) -> torch.Tensor:
    _dev(t, what)
    if t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{what} must hold {numel} elements for this call, not {t.numel()}")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, the call's other tensors on {device}")
    return t


def _nblocks(n: int, block: int):
    """Scale count of a flat call, or None when the library will refuse
    (n % block != 0 or an unsupported block: nothing is then dereferenced)."""
    if block not in BLOCK_SIZES or n % block:
        return None
    return n // block


def _expect_scales(t, what, nb, device):
    if nb is None:
        return _dev(t, what)
    return _expect(t, what, nb, (torch.float32,), device)


# ----------------------------------------------------------------------------
# the calls


# code formats: the C function suffix and the torch dtype that holds the codes
_INT8 = ("", torch.int8, 1)
_E4M3 = ("_e4m3", torch.uint8, 1)
_INT4 = ("_int4", torch.uint8, 2)          # two codes per byte


def _quantize(fmt, x, block, codes, scales, stream):
    name = "qar_quantize_blocks" + fmt[0]
    _dev(x, "x")
    n, dev = x.numel(), x.device
    nb = _nblocks(n, block)
    if codes is None:
        codes = torch.empty(n // fmt[2], dtype=fmt[1], device=dev)
    if scales is None:
        scales = torch.empty(max(n // block, 1) if block else 1, dtype=torch.float32, device=dev)
    if n:
        _expect(codes, "codes", n // fmt[2], _CODE_DTYPES, dev)
        _expect_scales(scales, "scales", nb, dev)
    _check(getattr(lib(), name)(x.data_ptr(), _dtype_code(x.dtype), n, block, _dev(codes, "codes").data_ptr(),
                                _dev(scales, "scales").data_ptr(), _stream(stream)), name)
    return codes, scales


def qar_quantize_blocks(x: torch.Tensor, block: int, codes: torch.Tensor | None = None,
                        scales: torch.Tensor | None = None, stream=None):
    """x (bf16/fp32, any shape, contiguous) -> (codes int8[n], scales fp32[n/block])."""
    return _quantize(_INT8, x, block, codes, scales, stream)


def qar_quantize_blocks_e4m3(x: torch.Tensor, block: int, codes: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None, stream=None):
    """x (bf16/fp32) -> (FP8 E4M3 codes uint8[n], scales fp32[n/block])."""
    return _quantize(_E4M3, x, block, codes, scales, stream)


def _out_args(out: torch.Tensor | None, n: int, device: torch.device):
    if out is None:
        return None, QAR_BF16
    if n:
        _expect(out, "out", n, _DATA_DTYPES, device)
    return _dev(out, "out").data_ptr(), _dtype_code(out.dtype)


def _expect_ranks(codes, scales, n, fmt, nb, device):
    """codes[r] / scales[r] of every rank: n elements' worth of codes and nb
    scales each, all on one device.  (A rank count above QAR_MAX_RANKS is
    left to the library, which refuses it before reading any pointer.)"""
    if len(codes) != len(scales) or not codes:
        raise ValueError("need one scales tensor per codes tensor, at least one rank")
    for r, (c, s) in enumerate(zip(codes, scales)):
        if n:
            _expect(c, f"codes[{r}]", n // fmt[2], _CODE_DTYPES, device)
            _expect_scales(s, f"scales[{r}]", nb, device)
        else:
            _dev(c, f"codes[{r}]"), _dev(s, f"scales[{r}]")


def _outputs(fmt, n, block, nb, codes_out, scales_out, dev):
    """codes_out / scales_out: allocated when not given, else checked."""
    if codes_out is None:
        codes_out = torch.empty(n // fmt[2], dtype=fmt[1], device=dev)
    elif n:
        _expect(codes_out, "codes_out", n // fmt[2], _CODE_DTYPES, dev)
    if scales_out is None:
        scales_out = torch.empty(max(n // block, 1) if block else 1, dtype=torch.float32, device=dev)
    elif n:
        _expect_scales(scales_out, "scales_out", nb, dev)
    return codes_out, scales_out


def _reduce(fmt, codes, scales, block, codes_out, scales_out, out, stream):
    name = "qar_reduce_quantized" + fmt[0]
    if len(codes) != len(scales) or not codes:
        raise ValueError("need one scales tensor per codes tensor, at least one rank")
    n = _dev(codes[0], "codes[0]").numel() * fmt[2]            # elements
    dev = codes[0].device
    nb = _nblocks(n, block)
    _expect_ranks(codes, scales, n, fmt, nb, dev)
    codes_out, scales_out = _outputs(fmt, n, block, nb, codes_out, scales_out, dev)
    optr, odt = _out_args(out, n, dev)
    cp, sp = _ptrs(codes), _ptrs(scales)
    _check(getattr(lib(), name)(ctypes.cast(cp, _vp), ctypes.cast(sp, _vp), len(codes), n, block,
                                _dev(codes_out, "codes_out").data_ptr(), _dev(scales_out, "scales_out").data_ptr(),
                                optr, odt, _stream(stream)), name)
    return codes_out, scales_out


def qar_reduce_quantized(codes: list[torch.Tensor], scales: list[torch.Tensor], block: int,
                         codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, stream=None):
    """One-shot N-way reduce of rank-ordered (codes, scales) -> (codes_out, scales_out);
    ``out`` (optional bf16/fp32 tensor) receives the dequantized result."""
    return _reduce(_INT8, codes, scales, block, codes_out, scales_out, out, stream)


def qar_quantize_blocks_int4(x: torch.Tensor, block: int, codes: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None, stream=None):
    """x (bf16/fp32) -> (4-bit codes packed two per byte, uint8[n/2]; scales fp32[n/block])."""
    return _quantize(_INT4, x, block, codes, scales, stream)


def qar_reduce_quantized_e4m3(codes: list[torch.Tensor], scales: list[torch.Tensor], block: int,
                              codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, stream=None):
    """The one-shot reduce with FP8 E4M3 codes (uint8 tensors)."""
    return _reduce(_E4M3, codes, scales, block, codes_out, scales_out, out, stream)


def _quantize_reduce(fmt, x_own, own, codes, scales, block, codes_out, scales_out, out, stream):
    name = "qar_quantize_reduce" + fmt[0]
    _dev(x_own, "x_own")
    n = x_own.numel()
    dev = x_own.device
    nb = _nblocks(n, block)
    _expect_ranks(codes, scales, n, fmt, nb, dev)
    codes_out, scales_out = _outputs(fmt, n, block, nb, codes_out, scales_out, dev)
    optr, odt = _out_args(out, n, dev)
    cp, sp = _ptrs(codes), _ptrs(scales)
    _check(getattr(lib(), name)(x_own.data_ptr(), _dtype_code(x_own.dtype), own, ctypes.cast(cp, _vp),
                                ctypes.cast(sp, _vp), len(codes), n, block, _dev(codes_out, "codes_out").data_ptr(),
                                _dev(scales_out, "scales_out").data_ptr(), optr, odt, _stream(stream)), name)
    return codes_out, scales_out


def qar_quantize_reduce(x_own: torch.Tensor, own: int, codes: list[torch.Tensor], scales: list[torch.Tensor],
                        block: int, codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, stream=None):
    """Quantize x_own into codes[own]/scales[own] and reduce all ranks in the
    same pass -> (codes_out, scales_out); ``out`` gets the dequantized result."""
    return _quantize_reduce(_INT8, x_own, own, codes, scales, block, codes_out, scales_out, out, stream)


def qar_reduce_quantized_int4(codes: list[torch.Tensor], scales: list[torch.Tensor], block: int,
                              codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, stream=None):
    """The one-shot reduce with packed 4-bit codes (uint8 tensors of n/2 bytes)."""
    return _reduce(_INT4, codes, scales, block, codes_out, scales_out, out, stream)


def qar_quantize_reduce_e4m3(x_own: torch.Tensor, own: int, codes: list[torch.Tensor],
                             scales: list[torch.Tensor], block: int, codes_out: torch.Tensor | None = None,
                             scales_out: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None):
    """The one-kernel step with FP8 E4M3 codes."""
    return _quantize_reduce(_E4M3, x_own, own, codes, scales, block, codes_out, scales_out, out, stream)


def qar_reduce_quantized_pipelined(codes: list[torch.Tensor], scales: list[torch.Tensor], block: int,
                                   nchunks: int, streams: list, codes_out: torch.Tensor | None = None,
                                   scales_out: torch.Tensor | None = None, out: torch.Tensor | None = None,
                                   stream=None):
    """The reduce cut into ``nchunks`` chunks enqueued round-robin on ``streams``."""
    if len(codes) != len(scales) or not codes:
        raise ValueError("need one scales tensor per codes tensor, at least one rank")
    n = _dev(codes[0], "codes[0]").numel()
    dev = codes[0].device
    nb = _nblocks(n, block)
    _expect_ranks(codes, scales, n, _INT8, nb, dev)
    codes_out, scales_out = _outputs(_INT8, n, block, nb, codes_out, scales_out, dev)
    optr, odt = _out_args(out, n, dev)
    cp, sp = _ptrs(codes), _ptrs(scales)
    sts = (ctypes.c_void_p * len(streams))(*[_stream(s) for s in streams])
    _check(lib().qar_reduce_quantized_pipelined(
        ctypes.cast(cp, _vp), ctypes.cast(sp, _vp), len(codes), n, block,
        _dev(codes_out, "codes_out").data_ptr(), _dev(scales_out, "scales_out").data_ptr(), optr, odt,
        nchunks, ctypes.cast(sts, _vp), len(streams), _stream(stream)), "qar_reduce_quantized_pipelined")
    return codes_out, scales_out


def qar_reduce_quantized_chunked(codes: list[torch.Tensor], scales: list[torch.Tensor], block: int, nchunks: int,
                                 streams: list, codes_out: torch.Tensor | None = None,
                                 scales_out: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The reduce cut into ``nchunks`` chunks (chunk c takes the runs c,
    c + nchunks, ... of QAR_CHUNK_RUN_ELEMS elements), chunk c enqueued on
    ``streams[c % len(streams)]`` behind that stream's earlier work, with no
    event or wait: the caller orders the streams."""
    if len(codes) != len(scales) or not codes:
        raise ValueError("need one scales tensor per codes tensor, at least one rank")
    n = _dev(codes[0], "codes[0]").numel()
    dev = codes[0].device
    nb = _nblocks(n, block)
    _expect_ranks(codes, scales, n, _INT8, nb, dev)
    codes_out, scales_out = _outputs(_INT8, n, block, nb, codes_out, scales_out, dev)
    optr, odt = _out_args(out, n, dev)
    cp, sp = _ptrs(codes), _ptrs(scales)
    sts = (ctypes.c_void_p * len(streams))(*[_stream(s) for s in streams])
    _check(lib().qar_reduce_quantized_chunked(
        ctypes.cast(cp, _vp), ctypes.cast(sp, _vp), len(codes), n, block,
        _dev(codes_out, "codes_out").data_ptr(), _dev(scales_out, "scales_out").data_ptr(), optr, odt,
        nchunks, ctypes.cast(sts, _vp), len(streams)), "qar_reduce_quantized_chunked")
    return codes_out, scales_out


def _ring_step(fmt, codes_in, scales_in, local, block, codes_out, scales_out, stream):
    name = "qar_ring_step" + fmt[0]
    _dev(local, "local")
    n, dev = local.numel(), local.device
    nb = _nblocks(n, block)
    if n:
        _expect(codes_in, "codes_in", n // fmt[2], _CODE_DTYPES, dev)
        _expect_scales(scales_in, "scales_in", nb, dev)
    _dev(codes_in, "codes_in"), _dev(scales_in, "scales_in")
    codes_out, scales_out = _outputs(fmt, n, block, nb, codes_out, scales_out, dev)
    _check(getattr(lib(), name)(codes_in.data_ptr(), scales_in.data_ptr(), local.data_ptr(),
                                _dtype_code(local.dtype), n, block, _dev(codes_out, "codes_out").data_ptr(),
                                _dev(scales_out, "scales_out").data_ptr(), _stream(stream)), name)
    return codes_out, scales_out


def qar_ring_step(codes_in: torch.Tensor, scales_in: torch.Tensor, local: torch.Tensor, block: int,
                  codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None, stream=None):
    """quantize(dequantize(codes_in, scales_in) + local) -> (codes_out, scales_out).
    Pass codes_out=codes_in, scales_out=scales_in to work in place."""
    return _ring_step(_INT8, codes_in, scales_in, local, block, codes_out, scales_out, stream)


def qar_quantize_reduce_int4(x_own: torch.Tensor, own: int, codes: list[torch.Tensor],
                             scales: list[torch.Tensor], block: int, codes_out: torch.Tensor | None = None,
                             scales_out: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None):
    """The one-kernel step with packed 4-bit codes."""
    return _quantize_reduce(_INT4, x_own, own, codes, scales, block, codes_out, scales_out, out, stream)


def qar_ring_step_e4m3(codes_in: torch.Tensor, scales_in: torch.Tensor, local: torch.Tensor, block: int,
                       codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None, stream=None):
    """The ring step with FP8 E4M3 codes."""
    return _ring_step(_E4M3, codes_in, scales_in, local, block, codes_out, scales_out, stream)


def _dequantize(fmt, codes, scales, block, out, out_dtype, stream):
    name = "qar_dequantize" + fmt[0]
    _dev(codes, "codes"), _dev(scales, "scales")
    n = codes.numel() * fmt[2]               # elements
    dev = codes.device
    if codes.dtype not in _CODE_DTYPES:
        raise TypeError(f"codes must be torch.int8 or torch.uint8, not {codes.dtype}")
    if n:
        _expect_scales(scales, "scales", _nblocks(n, block), dev)
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=dev)
    elif n:
        _expect(out, "out", n, _DATA_DTYPES, dev)
    _check(getattr(lib(), name)(codes.data_ptr(), scales.data_ptr(), n, block, _dev(out, "out").data_ptr(),
                                _dtype_code(out.dtype), _stream(stream)), name)
    return out


def qar_dequantize(codes: torch.Tensor, scales: torch.Tensor, block: int, out: torch.Tensor | None = None,
                   out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """codes, scales -> out (bf16 or fp32)."""
    return _dequantize(_INT8, codes, scales, block, out, out_dtype, stream)


def qar_ring_step_int4(codes_in: torch.Tensor, scales_in: torch.Tensor, local: torch.Tensor, block: int,
                       codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None, stream=None):
    """The ring step with packed 4-bit codes."""
    return _ring_step(_INT4, codes_in, scales_in, local, block, codes_out, scales_out, stream)


def qar_dequantize_e4m3(codes: torch.Tensor, scales: torch.Tensor, block: int, out: torch.Tensor | None = None,
                        out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """FP8 E4M3 codes (uint8), scales -> out (bf16 or fp32)."""
    return _dequantize(_E4M3, codes, scales, block, out, out_dtype, stream)


def qar_dequantize_int4(codes: torch.Tensor, scales: torch.Tensor, block: int, out: torch.Tensor | None = None,
                        out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Packed 4-bit codes (uint8, n/2 bytes), scales -> out (bf16 or fp32)."""
    return _dequantize(_INT4, codes, scales, block, out, out_dtype, stream)


def qar_reduce_unquantized(xs: list[torch.Tensor], out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The unquantized comparator: rank-order fp32 sum of N bf16/fp32 buffers."""
    if not xs:
        raise ValueError("need at least one rank")
    n, dt, dev = _dev(xs[0], "x[0]").numel(), xs[0].dtype, xs[0].device
    for r, x in enumerate(xs):
        _expect(x, f"x[{r}]", n, (dt,), dev)
    if out is None:
        out = torch.empty(n, dtype=dt, device=dev)
    else:
        _expect(out, "out", n, (dt,), dev)
    ptrs = _ptrs(xs)
    _check(lib().qar_reduce_unquantized(ctypes.cast(ptrs, _vp), len(xs), n, _dtype_code(xs[0].dtype),
                                        _dev(out, "out").data_ptr(), _stream(stream)), "qar_reduce_unquantized")
    return out


def qar_allreduce_simulated(xs: list[torch.Tensor], block: int, schedule: str = "one_shot", nchunks: int = 1,
                            streams: list | None = None, out: torch.Tensor | None = None,
                            workspace: tuple | None = None, stream=None) -> torch.Tensor:
    """The whole quantized AllReduce of N rank buffers on one GPU ('one_shot'
    or 'ring'); returns the dequantized result every rank would hold.
    ``workspace`` = (codes list, scales list) is allocated with torch when
    not given."""
    if not xs:
        raise ValueError("need at least one rank")
    sched = {"one_shot": QAR_SCHEDULE_ONE_SHOT, "ring": QAR_SCHEDULE_RING}[schedule]
    n, dt, dev = _dev(xs[0], "x[0]").numel(), xs[0].dtype, xs[0].device
    for r, x in enumerate(xs):
        _expect(x, f"x[{r}]", n, (dt,), dev)
    nwork = len(xs) if sched == QAR_SCHEDULE_ONE_SHOT else 1
    nb = _nblocks(n, block)
    if workspace is None:
        workspace = ([torch.empty(n, dtype=torch.int8, device=dev) for _ in range(nwork)],
                     [torch.empty(max(n // block, 1) if block else 1, dtype=torch.float32, device=dev)
                      for _ in range(nwork)])
    wc, ws = workspace
    if len(wc) < nwork or len(ws) < nwork:
        raise ValueError(f"the {schedule} schedule needs {nwork} codes and scales workspaces")
    wc, ws = list(wc)[:nwork], list(ws)[:nwork]
    if n:
        for r in range(nwork):
            _expect(wc[r], f"workspace codes[{r}]", n, _CODE_DTYPES, dev)
            _expect_scales(ws[r], f"workspace scales[{r}]", nb, dev)
    if out is None:
        out = torch.empty(n, dtype=dt, device=dev)
    else:
        _expect(out, "out", n, (dt,), dev)
    if streams is None:
        streams = [torch.cuda.current_stream()]
    xp, cp, sp = _ptrs(xs), _ptrs(wc), _ptrs(ws)
    sts = (ctypes.c_void_p * len(streams))(*[_stream(s) for s in streams])
    _check(lib().qar_allreduce_simulated(ctypes.cast(xp, _vp), _dtype_code(xs[0].dtype), len(xs), n, block, sched,
                                         ctypes.cast(cp, _vp), ctypes.cast(sp, _vp), _dev(out, "out").data_ptr(),
                                         nchunks, ctypes.cast(sts, _vp), len(streams), _stream(stream)),
           "qar_allreduce_simulated")
    return out


def qar_allreduce_simulated_static(xs: list[torch.Tensor], block: int, schedule: str = "one_shot",
                                   nchunks: int = 1, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """qar_allreduce_simulated on one stream with its staging in libqar's
    static device workspace (the library allocates nothing; ``out`` is
    allocated here with torch when not given)."""
    if not xs:
        raise ValueError("need at least one rank")
    sched = {"one_shot": QAR_SCHEDULE_ONE_SHOT, "ring": QAR_SCHEDULE_RING}[schedule]
    n, dt, dev = _dev(xs[0], "x[0]").numel(), xs[0].dtype, xs[0].device
    for r, x in enumerate(xs):
        _expect(x, f"x[{r}]", n, (dt,), dev)
    if out is None:
        out = torch.empty(n, dtype=dt, device=dev)
    else:
        _expect(out, "out", n, (dt,), dev)
    xp = _ptrs(xs)
    _check(lib().qar_allreduce_simulated_static(ctypes.cast(xp, _vp), _dtype_code(dt), len(xs), n, block, sched,
                                                out.data_ptr(), nchunks, _stream(stream)),
           "qar_allreduce_simulated_static")
    return out


# ----------------------------------------------------------------------------
# row-bounded blocks ([rows, row_len] tensors; the block grid restarts per row)


def row_blocks(rows: int, row_len: int, block: int) -> int:
    return rows * (-(-row_len // block))


def _row_nblocks(rows: int, row_len: int, block: int):
    """Scale count of a row-bounded call, or None for a block size the
    library refuses."""
    return row_blocks(rows, row_len, block) if block in BLOCK_SIZES else None


def qar_quantize_rows(x: torch.Tensor, block: int, codes: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None, stream=None):
    """x: [rows, row_len] bf16/fp32 -> (codes [rows*row_len], scales [rows*ceil(row_len/block)])."""
    _dev(x, "x")
    rows, row_len = x.shape
    dev = x.device
    nrb = _row_nblocks(rows, row_len, block)
    if codes is None:
        codes = torch.empty(rows * row_len, dtype=torch.int8, device=dev)
    elif rows * row_len:
        _expect(codes, "codes", rows * row_len, _CODE_DTYPES, dev)
    if scales is None:
        scales = torch.empty(max(nrb or 0, 1), dtype=torch.float32, device=dev)
    elif rows * row_len:
        _expect_scales(scales, "scales", nrb, dev)
    _check(lib().qar_quantize_rows(x.data_ptr(), _dtype_code(x.dtype), rows, row_len, block,
                                   _dev(codes, "codes").data_ptr(), _dev(scales, "scales").data_ptr(),
                                   _stream(stream)), "qar_quantize_rows")
    return codes, scales


def qar_reduce_quantized_rows(codes: list[torch.Tensor], scales: list[torch.Tensor], rows: int, row_len: int,
                              block: int, codes_out: torch.Tensor | None = None,
                              scales_out: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None):
    if len(codes) != len(scales) or not codes:
        raise ValueError("need one scales tensor per codes tensor, at least one rank")
    n = rows * row_len
    dev = _dev(codes[0], "codes[0]").device
    nrb = _row_nblocks(rows, row_len, block)
    _expect_ranks(codes, scales, n, _INT8, nrb, dev)
    if codes_out is None:
        codes_out = torch.empty(n, dtype=torch.int8, device=dev)
    elif n:
        _expect(codes_out, "codes_out", n, _CODE_DTYPES, dev)
    if scales_out is None:
        scales_out = torch.empty(max(nrb or 0, 1), dtype=torch.float32, device=dev)
    elif n:
        _expect_scales(scales_out, "scales_out", nrb, dev)
    optr, odt = _out_args(out, n, dev)
    cp, sp = _ptrs(codes), _ptrs(scales)
    _check(lib().qar_reduce_quantized_rows(ctypes.cast(cp, _vp), ctypes.cast(sp, _vp), len(codes), rows, row_len,
                                           block, _dev(codes_out, "codes_out").data_ptr(),
                                           _dev(scales_out, "scales_out").data_ptr(), optr, odt, _stream(stream)),
           "qar_reduce_quantized_rows")
    return codes_out, scales_out


def qar_ring_step_rows(codes_in: torch.Tensor, scales_in: torch.Tensor, local: torch.Tensor, block: int,
                       codes_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None, stream=None):
    """local: [rows, row_len]; codes/scales in the row-bounded layout."""
    _dev(codes_in, "codes_in"), _dev(scales_in, "scales_in"), _dev(local, "local")
    rows, row_len = local.shape
    n, dev = rows * row_len, local.device
    nrb = _row_nblocks(rows, row_len, block)
    if n:
        _expect(codes_in, "codes_in", n, _CODE_DTYPES, dev)
        _expect_scales(scales_in, "scales_in", nrb, dev)
    if codes_out is None:
        codes_out = torch.empty(n, dtype=torch.int8, device=dev)
    elif n:
        _expect(codes_out, "codes_out", n, _CODE_DTYPES, dev)
    if scales_out is None:
        scales_out = torch.empty(max(nrb or 0, 1), dtype=torch.float32, device=dev)
    elif n:
        _expect_scales(scales_out, "scales_out", nrb, dev)
    _check(lib().qar_ring_step_rows(codes_in.data_ptr(), scales_in.data_ptr(), local.data_ptr(),
                                    _dtype_code(local.dtype), rows, row_len, block,
                                    _dev(codes_out, "codes_out").data_ptr(), _dev(scales_out, "scales_out").data_ptr(),
                                    _stream(stream)), "qar_ring_step_rows")
    return codes_out, scales_out


def qar_dequantize_rows(codes: torch.Tensor, scales: torch.Tensor, rows: int, row_len: int, block: int,
                        out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                        stream=None) -> torch.Tensor:
    _dev(codes, "codes"), _dev(scales, "scales")
    n, dev = rows * row_len, codes.device
    if n:
        _expect(codes, "codes", n, _CODE_DTYPES, dev)
        _expect_scales(scales, "scales", _row_nblocks(rows, row_len, block), dev)
    if out is None:
        out = torch.empty(rows, row_len, dtype=out_dtype, device=dev)
    elif n:
        _expect(out, "out", n, _DATA_DTYPES, dev)
    _check(lib().qar_dequantize_rows(codes.data_ptr(), scales.data_ptr(), rows, row_len, block,
                                     _dev(out, "out").data_ptr(), _dtype_code(out.dtype), _stream(stream)),
           "qar_dequantize_rows")
    return out
