"""Plain CPU oracle for dynamic block-wise int8 quantized reduction.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library package.

The arithmetic lives in ``qar_oracle.c`` (plain scalar C, one IEEE binary32
rounding per operation).  This module only compiles it with gcc, loads it with
ctypes and moves numpy arrays in and out.  bf16 data travels as ``uint16``
bit patterns.

Method: "EQuARX: Efficient Quantized AllReduce in XLA for Distributed Machine
Learning Acceleration" -- page summary, section "technical framework" steps
1-4 (blocking, dynamic per-block quantization to INT8, AllReduce on the
quantized data, dequantization to the original type) and section "key
design" item 1 (per-block range found at run time).  The C file's header
lists the readings of the open points.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qar_oracle.c")
LIBRARY = os.path.join(_HERE, "libqar_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

BF16 = 0
F32 = 1


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc into ``output``; returns its path."""
    tmp = output + ".tmp"
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes view of one compiled oracle shared object."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.oracle_quantize.argtypes = [vp, ctypes.c_int, sz, sz, vp, vp]
        lib.oracle_dequantize_f32.argtypes = [vp, vp, sz, sz, vp]
        lib.oracle_dequantize_bf16.argtypes = [vp, vp, sz, sz, vp]
        lib.oracle_reduce.argtypes = [vp, vp, sz, sz, sz, vp, vp]
        lib.oracle_ring_step.argtypes = [vp, vp, vp, ctypes.c_int, sz, sz, vp, vp]
        lib.oracle_reduce_unquantized.argtypes = [vp, ctypes.c_int, sz, sz, vp]
        lib.oracle_f32_to_bf16.argtypes = [vp, sz, vp]
        lib.oracle_f32_to_bf16.restype = None
        lib.oracle_quantize_e4m3.argtypes = [vp, ctypes.c_int, sz, sz, vp, vp]
        lib.oracle_dequantize_e4m3.argtypes = [vp, vp, sz, sz, ctypes.c_int, vp]
        lib.oracle_reduce_e4m3.argtypes = [vp, vp, sz, sz, sz, vp, vp]
        lib.oracle_ring_step_e4m3.argtypes = [vp, vp, vp, ctypes.c_int, sz, sz, vp, vp]
        lib.oracle_e4m3_encode.argtypes = [vp, sz, vp]
        lib.oracle_e4m3_encode.restype = None
        lib.oracle_e4m3_decode.argtypes = [vp, sz, vp]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_quantize_int4.argtypes = [vp, ctypes.c_int, sz, sz, vp, vp]
        lib.oracle_dequantize_int4.argtypes = [vp, vp, sz, sz, ctypes.c_int, vp]
        lib.oracle_reduce_int4.argtypes = [vp, vp, sz, sz, sz, vp, vp]
        lib.oracle_ring_step_int4.argtypes = [vp, vp, vp, ctypes.c_int, sz, sz, vp, vp]
        for name in ("oracle_quantize", "oracle_dequantize_f32", "oracle_dequantize_bf16",
                     "oracle_reduce", "oracle_ring_step", "oracle_reduce_unquantized",
                     "oracle_quantize_e4m3", "oracle_dequantize_e4m3", "oracle_reduce_e4m3",
                     "oracle_ring_step_e4m3", "oracle_quantize_int4", "oracle_dequantize_int4",
                     "oracle_reduce_int4", "oracle_ring_step_int4"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib

    # -- helpers --------------------------------------------------------
    @staticmethod
    def _dtype_of(x: np.ndarray) -> int:
        if x.dtype == np.uint16:
            return BF16
        if x.dtype == np.float32:
            return F32
        raise TypeError(f"oracle inputs are bf16 bit patterns (uint16) or float32, got {x.dtype}")

    @staticmethod
    def _ptr(a: np.ndarray) -> int:
        return a.ctypes.data

    @staticmethod
    def _check(rc: int, what: str) -> None:
        if rc == -2:
            raise ValueError(f"{what}: non-finite input")
        if rc != 0:
            raise ValueError(f"{what}: bad argument (rc={rc})")

    @staticmethod
    def nblocks(n: int, block: int) -> int:
        return (n + block - 1) // block

    # -- the method -----------------------------------------------------
    def quantize(self, x: np.ndarray, block: int):
        """x (bf16 uint16 patterns or float32, 1-D) -> (codes int8[n], scales float32[nb])."""
        x = np.ascontiguousarray(x).reshape(-1)
        n = x.size
        codes = np.empty(n, np.int8)
        scales = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_quantize(self._ptr(x), self._dtype_of(x), n, block,
                                      self._ptr(codes), self._ptr(scales))
        self._check(rc, "quantize")
        return codes, scales

    def dequantize(self, codes: np.ndarray, scales: np.ndarray, block: int, out: str = "f32"):
        """codes, scales -> float32[n] (out='f32') or bf16 uint16 patterns (out='bf16')."""
        codes = np.ascontiguousarray(codes, np.int8).reshape(-1)
        scales = np.ascontiguousarray(scales, np.float32).reshape(-1)
        n = codes.size
        if scales.size < self.nblocks(n, block):
            raise ValueError("too few scales")
        if out == "f32":
            res = np.empty(n, np.float32)
            rc = self.lib.oracle_dequantize_f32(self._ptr(codes), self._ptr(scales), n, block,
                                                self._ptr(res))
        elif out == "bf16":
            res = np.empty(n, np.uint16)
            rc = self.lib.oracle_dequantize_bf16(self._ptr(codes), self._ptr(scales), n, block,
                                                 self._ptr(res))
        else:
            raise ValueError(out)
        self._check(rc, "dequantize")
        return res

    def reduce(self, codes: list, scales: list, block: int):
        """One-shot N-way reduce over rank-ordered (codes, scales) -> (codes, scales)."""
        nranks = len(codes)
        if nranks == 0 or nranks != len(scales):
            raise ValueError("need one scales array per codes array, at least one rank")
        codes = [np.ascontiguousarray(c, np.int8).reshape(-1) for c in codes]
        scales = [np.ascontiguousarray(s, np.float32).reshape(-1) for s in scales]
        n = codes[0].size
        nb = self.nblocks(n, block)
        for c, s in zip(codes, scales):
            if c.size != n or s.size < nb:
                raise ValueError("rank buffers differ in size")
        cptr = (ctypes.c_void_p * nranks)(*[self._ptr(c) for c in codes])
        sptr = (ctypes.c_void_p * nranks)(*[self._ptr(s) for s in scales])
        out_c = np.empty(n, np.int8)
        out_s = np.empty(nb, np.float32)
        rc = self.lib.oracle_reduce(ctypes.cast(cptr, ctypes.c_void_p),
                                    ctypes.cast(sptr, ctypes.c_void_p),
                                    nranks, n, block, self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "reduce")
        return out_c, out_s

    def ring_step(self, codes_in: np.ndarray, scales_in: np.ndarray, local: np.ndarray, block: int):
        """quantize(dequantize(codes_in, scales_in) + local) -> (codes, scales)."""
        codes_in = np.ascontiguousarray(codes_in, np.int8).reshape(-1)
        scales_in = np.ascontiguousarray(scales_in, np.float32).reshape(-1)
        local = np.ascontiguousarray(local).reshape(-1)
        n = codes_in.size
        if local.size != n or scales_in.size < self.nblocks(n, block):
            raise ValueError("size mismatch")
        out_c = np.empty(n, np.int8)
        out_s = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_ring_step(self._ptr(codes_in), self._ptr(scales_in), self._ptr(local),
                                       self._dtype_of(local), n, block,
                                       self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "ring_step")
        return out_c, out_s

    def reduce_unquantized(self, xs: list) -> np.ndarray:
        """Rank-order fp32 sum of N unquantized buffers, in their own dtype."""
        xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
        if not xs:
            raise ValueError("need at least one rank")
        dt = self._dtype_of(xs[0])
        n = xs[0].size
        for x in xs:
            if x.size != n or self._dtype_of(x) != dt:
                raise ValueError("rank buffers differ in size or type")
        ptrs = (ctypes.c_void_p * len(xs))(*[self._ptr(x) for x in xs])
        out = np.empty(n, xs[0].dtype)
        rc = self.lib.oracle_reduce_unquantized(ctypes.cast(ptrs, ctypes.c_void_p), dt, len(xs), n,
                                                self._ptr(out))
        self._check(rc, "reduce_unquantized")
        return out

    def f32_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, np.float32).reshape(-1)
        out = np.empty(x.size, np.uint16)
        self.lib.oracle_f32_to_bf16(self._ptr(x), x.size, self._ptr(out))
        return out

    # -- FP8 E4M3 codes -------------------------------------------------
    def quantize_e4m3(self, x: np.ndarray, block: int):
        """x (bf16 uint16 patterns or float32) -> (E4M3 codes uint8[n], scales float32[nb])."""
        x = np.ascontiguousarray(x).reshape(-1)
        n = x.size
        codes = np.empty(n, np.uint8)
        scales = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_quantize_e4m3(self._ptr(x), self._dtype_of(x), n, block,
                                           self._ptr(codes), self._ptr(scales))
        self._check(rc, "quantize_e4m3")
        return codes, scales

    def dequantize_e4m3(self, codes: np.ndarray, scales: np.ndarray, block: int, out: str = "f32"):
        codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
        scales = np.ascontiguousarray(scales, np.float32).reshape(-1)
        n = codes.size
        if scales.size < self.nblocks(n, block):
            raise ValueError("too few scales")
        if out not in ("f32", "bf16"):
            raise ValueError(out)
        res = np.empty(n, np.float32 if out == "f32" else np.uint16)
        rc = self.lib.oracle_dequantize_e4m3(self._ptr(codes), self._ptr(scales), n, block,
                                             F32 if out == "f32" else BF16, self._ptr(res))
        self._check(rc, "dequantize_e4m3")
        return res

    def reduce_e4m3(self, codes: list, scales: list, block: int):
        nranks = len(codes)
        if nranks == 0 or nranks != len(scales):
            raise ValueError("need one scales array per codes array, at least one rank")
        codes = [np.ascontiguousarray(c, np.uint8).reshape(-1) for c in codes]
        scales = [np.ascontiguousarray(s, np.float32).reshape(-1) for s in scales]
        n = codes[0].size
        nb = self.nblocks(n, block)
        for c, s in zip(codes, scales):
            if c.size != n or s.size < nb:
                raise ValueError("rank buffers differ in size")
        cptr = (ctypes.c_void_p * nranks)(*[self._ptr(c) for c in codes])
        sptr = (ctypes.c_void_p * nranks)(*[self._ptr(s) for s in scales])
        out_c = np.empty(n, np.uint8)
        out_s = np.empty(nb, np.float32)
        rc = self.lib.oracle_reduce_e4m3(ctypes.cast(cptr, ctypes.c_void_p), ctypes.cast(sptr, ctypes.c_void_p),
                                         nranks, n, block, self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "reduce_e4m3")
        return out_c, out_s

    def ring_step_e4m3(self, codes_in: np.ndarray, scales_in: np.ndarray, local: np.ndarray, block: int):
        codes_in = np.ascontiguousarray(codes_in, np.uint8).reshape(-1)
        scales_in = np.ascontiguousarray(scales_in, np.float32).reshape(-1)
        local = np.ascontiguousarray(local).reshape(-1)
        n = codes_in.size
        if local.size != n or scales_in.size < self.nblocks(n, block):
            raise ValueError("size mismatch")
        out_c = np.empty(n, np.uint8)
        out_s = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_ring_step_e4m3(self._ptr(codes_in), self._ptr(scales_in), self._ptr(local),
                                            self._dtype_of(local), n, block, self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "ring_step_e4m3")
        return out_c, out_s

    def e4m3_encode(self, x: np.ndarray) -> np.ndarray:
        """float32 values with |x| <= 448 -> nearest E4M3 codes (ties to even)."""
        x = np.ascontiguousarray(x, np.float32).reshape(-1)
        if np.any(np.abs(x) > 448.0) or not np.all(np.isfinite(x)):
            raise ValueError("e4m3_encode takes finite values within [-448, 448]")
        out = np.empty(x.size, np.uint8)
        self.lib.oracle_e4m3_encode(self._ptr(x), x.size, self._ptr(out))
        return out

    def e4m3_decode(self, c: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(c, np.uint8).reshape(-1)
        out = np.empty(c.size, np.float32)
        self.lib.oracle_e4m3_decode(self._ptr(c), c.size, self._ptr(out))
        return out

    # -- 4-bit integer codes, two per byte --------------------------------
    @staticmethod
    def int4_bytes(n: int) -> int:
        return (n + 1) // 2

    def quantize_int4(self, x: np.ndarray, block: int):
        """x -> (packed codes uint8[ceil(n/2)], scales float32[nb])."""
        x = np.ascontiguousarray(x).reshape(-1)
        n = x.size
        codes = np.zeros(self.int4_bytes(n), np.uint8)
        scales = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_quantize_int4(self._ptr(x), self._dtype_of(x), n, block, self._ptr(codes),
                                           self._ptr(scales))
        self._check(rc, "quantize_int4")
        return codes, scales

    def dequantize_int4(self, codes: np.ndarray, scales: np.ndarray, block: int, n: int, out: str = "f32"):
        codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
        scales = np.ascontiguousarray(scales, np.float32).reshape(-1)
        if codes.size < self.int4_bytes(n) or scales.size < self.nblocks(n, block):
            raise ValueError("too few codes or scales")
        if out not in ("f32", "bf16"):
            raise ValueError(out)
        res = np.empty(n, np.float32 if out == "f32" else np.uint16)
        rc = self.lib.oracle_dequantize_int4(self._ptr(codes), self._ptr(scales), n, block,
                                             F32 if out == "f32" else BF16, self._ptr(res))
        self._check(rc, "dequantize_int4")
        return res

    def reduce_int4(self, codes: list, scales: list, block: int, n: int):
        nranks = len(codes)
        if nranks == 0 or nranks != len(scales):
            raise ValueError("need one scales array per codes array, at least one rank")
        codes = [np.ascontiguousarray(c, np.uint8).reshape(-1) for c in codes]
        scales = [np.ascontiguousarray(s, np.float32).reshape(-1) for s in scales]
        nb = self.nblocks(n, block)
        for c, s in zip(codes, scales):
            if c.size < self.int4_bytes(n) or s.size < nb:
                raise ValueError("rank buffers too small")
        cptr = (ctypes.c_void_p * nranks)(*[self._ptr(c) for c in codes])
        sptr = (ctypes.c_void_p * nranks)(*[self._ptr(s) for s in scales])
        out_c = np.zeros(self.int4_bytes(n), np.uint8)
        out_s = np.empty(nb, np.float32)
        rc = self.lib.oracle_reduce_int4(ctypes.cast(cptr, ctypes.c_void_p), ctypes.cast(sptr, ctypes.c_void_p),
                                         nranks, n, block, self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "reduce_int4")
        return out_c, out_s

    def ring_step_int4(self, codes_in: np.ndarray, scales_in: np.ndarray, local: np.ndarray, block: int):
        local = np.ascontiguousarray(local).reshape(-1)
        n = local.size
        codes_in = np.ascontiguousarray(codes_in, np.uint8).reshape(-1)
        scales_in = np.ascontiguousarray(scales_in, np.float32).reshape(-1)
        if codes_in.size < self.int4_bytes(n) or scales_in.size < self.nblocks(n, block):
            raise ValueError("size mismatch")
        out_c = np.zeros(self.int4_bytes(n), np.uint8)
        out_s = np.empty(self.nblocks(n, block), np.float32)
        rc = self.lib.oracle_ring_step_int4(self._ptr(codes_in), self._ptr(scales_in), self._ptr(local),
                                            self._dtype_of(local), n, block, self._ptr(out_c), self._ptr(out_s))
        self._check(rc, "ring_step_int4")
        return out_c, out_s


_default = None


def load() -> Oracle:
    """The oracle built from ``qar_oracle.c``; compiled first if not built yet."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
