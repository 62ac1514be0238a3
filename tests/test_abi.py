"""The C ABI without a GPU: libqar loads, exports every function
include/qar.h declares, and rejects bad arguments before touching HIP (every
call below fails validation, so nothing is launched)."""
import ctypes

import pytest

from block_wise_int8_amd import qar


@pytest.fixture(scope="module")
def L():
    return qar.lib()


def test_exports_every_declared_function(L):
    names = qar.declared_functions()
    assert set(names) == set(qar._SIGNATURES), names
    for name in names:
        assert hasattr(L, name), name


def test_binding_constants_match_the_header():
    """The binding's copies of the header's limits and sizes."""
    import re
    text = open(qar.HEADER).read()

    def define(name):
        m = re.search(rf"^#define {name} ([^\n]+?)\s*$", text, re.M)
        assert m, name
        expr = re.sub(r"(\d)u\b", r"\1", m.group(1).replace("(size_t)", ""))
        assert re.fullmatch(r"[\d\s()<]+", expr), expr          # integers, parentheses and shifts only
        return eval(expr, {})
    for name in ("QAR_MAX_RANKS", "QAR_MAX_STREAMS", "QAR_STATIC_WORKSPACE_BYTES", "QAR_CHUNK_RUN_ELEMS"):
        assert define(name) == getattr(qar, name), name


def test_status_strings(L):
    for s in range(6):
        assert L.qar_status_string(s)
    assert L.qar_last_error() == b""


A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
B_ = 0x20000
C = 0x30000
D = 0x40000


def test_quantize_validation(L):
    q = L.qar_quantize_blocks
    assert q(None, qar.QAR_BF16, 0, 256, None, None, None) == qar.QAR_OK           # empty call
    assert q(None, qar.QAR_BF16, 256, 256, B_, C, None) == qar.QAR_ERR_INVALID_ARG
    assert q(A, qar.QAR_BF16, 256, 100, B_, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert q(A, qar.QAR_BF16, 300, 256, B_, C, None) == qar.QAR_ERR_INVALID_ARG   # n % block
    assert q(A, 7, 256, 256, B_, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert q(A + 2, qar.QAR_BF16, 256, 256, B_, C, None) == qar.QAR_ERR_MISALIGNED
    assert q(A, qar.QAR_BF16, 256, 256, B_ + 8, C, None) == qar.QAR_ERR_MISALIGNED
    assert q(A, qar.QAR_BF16, 256, 256, B_, C + 2, None) == qar.QAR_ERR_MISALIGNED
    assert q(A, qar.QAR_BF16, 256, 256, A + 256, C, None) == qar.QAR_ERR_INVALID_ARG  # codes overlap x
    assert q(A, qar.QAR_BF16, (1 << 40) + 256, 256, B_, C, None) == qar.QAR_ERR_INVALID_ARG


def _arr(*v):
    return ctypes.cast((ctypes.c_void_p * len(v))(*v), ctypes.c_void_p)


def test_reduce_validation(L):
    r = L.qar_reduce_quantized
    codes, scales = _arr(A, B_), _arr(C, D)
    assert r(None, None, 2, 0, 256, None, None, None, 0, None) == qar.QAR_OK
    assert r(codes, scales, 0, 256, 256, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    assert r(codes, scales, 33, 256, 256, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    assert r(codes, scales, 2, 256, 64 * 3, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_UNSUPPORTED
    assert r(_arr(A, B_ + 1), scales, 2, 256, 256, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_MISALIGNED
    assert r(_arr(A, None), scales, 2, 256, 256, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    # output codes partly overlapping rank 1's codes
    assert r(codes, scales, 2, 256, 256, B_ + 16, 0x60000, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    # in place on codes but not on scales
    assert r(codes, scales, 2, 256, 256, B_, 0x60000, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    # optional output with a bad dtype
    assert r(codes, scales, 2, 256, 256, 0x50000, 0x60000, 0x70000, 9, None) == qar.QAR_ERR_UNSUPPORTED


def test_quantize_reduce_validation(L):
    r = L.qar_quantize_reduce
    X = 0x80000
    codes, scales = _arr(A, B_), _arr(C, D)
    ok = (codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, None)
    assert r(None, 0, 0, None, None, 2, 0, 256, None, None, None, 0, None) == qar.QAR_OK
    assert r(None, 0, 0, *ok) == qar.QAR_ERR_INVALID_ARG
    assert r(X, 7, 0, *ok) == qar.QAR_ERR_UNSUPPORTED                        # input dtype
    assert r(X, 0, 2, *ok) == qar.QAR_ERR_INVALID_ARG                        # own >= nranks
    assert r(X + 2, 0, 0, *ok) == qar.QAR_ERR_MISALIGNED
    assert r(X, 0, 0, codes, scales, 2, 256, 96, 0x50000, 0x60000, None, 0, None) == qar.QAR_ERR_UNSUPPORTED
    # rank own's codes (an output) may not be the result's codes, even in place
    assert r(X, 0, 1, codes, scales, 2, 256, 256, B_, D, None, 0, None) == qar.QAR_ERR_INVALID_ARG
    # the input may not overlap rank own's codes or the result
    assert r(A + 128, 0, 0, *ok) == qar.QAR_ERR_INVALID_ARG
    assert r(0x50000, 0, 0, *ok) == qar.QAR_ERR_INVALID_ARG
    assert r(X, 0, 0, codes, scales, 2, 256, 256, 0x50000, 0x60000, X + 64, 0, None) == qar.QAR_ERR_INVALID_ARG
    # rank own's codes overlapping another rank's scales
    assert r(X, 0, 0, _arr(A, B_), _arr(A + 64, D), 2, 256, 256, 0x50000, 0x60000, None, 0, None) \
        == qar.QAR_ERR_INVALID_ARG


def test_e4m3_validation(L):
    """The E4M3 calls share the int8 calls' checks."""
    codes, scales = _arr(A, B_), _arr(C, D)
    assert L.qar_quantize_blocks_e4m3(A, 0, 0, 256, B_, C, None) == qar.QAR_OK
    assert L.qar_quantize_blocks_e4m3(A, 0, 256, 96, B_, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert L.qar_quantize_blocks_e4m3(A + 2, 0, 256, 256, B_, C, None) == qar.QAR_ERR_MISALIGNED
    assert L.qar_quantize_blocks_e4m3(A, 0, 256, 256, A + 64, C, None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_reduce_quantized_e4m3(codes, scales, 33, 256, 256, 0x50000, 0x60000, None, 0, None) \
        == qar.QAR_ERR_INVALID_ARG
    assert L.qar_reduce_quantized_e4m3(codes, scales, 2, 256, 256, B_ + 16, 0x60000, None, 0, None) \
        == qar.QAR_ERR_INVALID_ARG
    assert L.qar_quantize_reduce_e4m3(0x80000, 0, 2, codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0,
                                      None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_ring_step_e4m3(A, C, 0x80000, 0, 256, 256, A, 0x60000, None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_dequantize_e4m3(A, C, 256, 256, A + 16, 0, None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_dequantize_e4m3(A, C, 256, 256, 0x80000, 5, None) == qar.QAR_ERR_UNSUPPORTED


def test_int4_validation(L):
    """4-bit code buffers hold n/2 bytes, and overlaps are judged on that
    size.  Every call here fails a check, so nothing is launched."""
    codes, scales = _arr(A, B_), _arr(C, D + 2)        # rank 1's scales misaligned
    # codes_out 128 bytes after rank 0's codes: adjacent at n/2 = 128 bytes, so
    # the check reaches rank 1 and reports its misaligned scales (with n bytes
    # of codes it would have been an overlap)
    assert L.qar_reduce_quantized_int4(codes, scales, 2, 256, 256, A + 128, 0x60000, None, 0, None) \
        == qar.QAR_ERR_MISALIGNED
    assert L.qar_reduce_quantized(codes, scales, 2, 256, 256, A + 128, 0x60000, None, 0, None) \
        == qar.QAR_ERR_INVALID_ARG
    # 64 bytes after: an overlap for 4-bit codes too
    assert L.qar_reduce_quantized_int4(codes, scales, 2, 256, 256, A + 64, 0x60000, None, 0, None) \
        == qar.QAR_ERR_INVALID_ARG
    assert L.qar_quantize_blocks_int4(A, 0, 256, 96, B_, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert L.qar_quantize_blocks_int4(A, 0, 256, 256, A + 256, C, None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_ring_step_int4(A, C, 0x80000, 0, 256, 96, B_, D, None) == qar.QAR_ERR_UNSUPPORTED
    assert L.qar_dequantize_int4(A, C, 256, 256, A + 64, 0, None) == qar.QAR_ERR_INVALID_ARG
    assert L.qar_quantize_reduce_int4(0x80000, 0, 2, _arr(A, B_), _arr(C, D), 2, 256, 256, 0x50000, 0x60000,
                                      None, 0, None) == qar.QAR_ERR_INVALID_ARG


def test_pipelined_validation(L):
    p = L.qar_reduce_quantized_pipelined
    codes, scales = _arr(A, B_), _arr(C, D)
    streams = _arr(0x1234)
    assert p(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 0, streams, 1, None) == qar.QAR_ERR_INVALID_ARG
    assert p(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, streams, 0, None) == qar.QAR_ERR_INVALID_ARG
    assert p(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, None, 1, None) == qar.QAR_ERR_INVALID_ARG
    assert p(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, streams, 17, None) == qar.QAR_ERR_INVALID_ARG
    # the default stream (NULL) may stand in streams[] only as the calling stream itself
    assert p(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, _arr(None), 1, 0x9999) == \
        qar.QAR_ERR_INVALID_ARG


def test_ring_and_dequantize_validation(L):
    g = L.qar_ring_step
    assert g(A, C, B_, qar.QAR_BF16, 0, 256, A, C, None) == qar.QAR_OK
    assert g(A, C, B_, qar.QAR_BF16, 256, 32, A, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert g(A, C, B_, qar.QAR_BF16, 256, 256, A, D, None) == qar.QAR_ERR_INVALID_ARG   # half in place
    assert g(A, C, B_, qar.QAR_BF16, 256, 256, B_ + 64, D, None) == qar.QAR_ERR_INVALID_ARG  # codes_out overlaps local
    assert g(A, C, B_ + 4, qar.QAR_F32, 256, 256, A, C, None) == qar.QAR_ERR_MISALIGNED
    d = L.qar_dequantize
    assert d(A, C, 0, 256, None, qar.QAR_F32, None) == qar.QAR_OK
    assert d(A, C, 512, 256, None, qar.QAR_F32, None) == qar.QAR_ERR_INVALID_ARG
    assert d(A, C, 512, 256, A + 64, qar.QAR_F32, None) == qar.QAR_ERR_INVALID_ARG    # out overlaps codes
    assert d(A, C, 512, 256, D, 5, None) == qar.QAR_ERR_UNSUPPORTED
    assert d(A, C, 500, 256, D, qar.QAR_F32, None) == qar.QAR_ERR_INVALID_ARG


def test_unquantized_validation(L):
    u = L.qar_reduce_unquantized
    xs = _arr(A, B_)
    assert u(None, 2, 0, qar.QAR_BF16, None, None) == qar.QAR_OK
    assert u(xs, 0, 256, qar.QAR_BF16, C, None) == qar.QAR_ERR_INVALID_ARG
    assert u(xs, 33, 256, qar.QAR_BF16, C, None) == qar.QAR_ERR_INVALID_ARG
    assert u(xs, 2, 250, qar.QAR_BF16, C, None) == qar.QAR_ERR_INVALID_ARG       # n % 16
    assert u(xs, 2, 256, 4, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert u(xs, 2, 256, qar.QAR_BF16, C + 8, None) == qar.QAR_ERR_MISALIGNED
    assert u(_arr(A, B_ + 2), 2, 256, qar.QAR_BF16, C, None) == qar.QAR_ERR_MISALIGNED
    assert u(_arr(A, None), 2, 256, qar.QAR_BF16, C, None) == qar.QAR_ERR_INVALID_ARG
    assert u(xs, 2, 256, qar.QAR_BF16, A + 32, None) == qar.QAR_ERR_INVALID_ARG    # partial overlap


def test_allreduce_simulated_validation(L):
    f = L.qar_allreduce_simulated
    xs, cw, sw, st = _arr(A, B_), _arr(C, D), _arr(0x50000, 0x60000), _arr(0x1234)
    ok_args = (xs, qar.QAR_BF16, 2, 256, 256, qar.QAR_SCHEDULE_ONE_SHOT, cw, sw, 0x70000, 1, st, 1, None)
    assert f(xs, qar.QAR_BF16, 2, 0, 256, 0, cw, sw, 0x70000, 1, st, 1, None) == qar.QAR_OK
    bad = list(ok_args); bad[5] = 7
    assert f(*bad) == qar.QAR_ERR_UNSUPPORTED                       # schedule
    bad = list(ok_args); bad[9] = 0
    assert f(*bad) == qar.QAR_ERR_INVALID_ARG                       # nchunks
    bad = list(ok_args); bad[8] = B_ + 64
    assert f(*bad) == qar.QAR_ERR_INVALID_ARG                       # out overlaps an input
    bad = list(ok_args); bad[6] = _arr(C, C + 128)
    assert f(*bad) == qar.QAR_ERR_INVALID_ARG                       # workspaces overlap
    bad = list(ok_args); bad[6] = _arr(C, None)
    assert f(*bad) == qar.QAR_ERR_INVALID_ARG                       # one-shot needs every rank's workspace
    bad = list(ok_args); bad[5] = qar.QAR_SCHEDULE_RING; bad[6] = _arr(C, None); bad[7] = _arr(0x50000, None)
    bad[8] = 0x70001
    assert f(*bad) == qar.QAR_ERR_MISALIGNED                        # ring needs only [0]; out misaligned


def test_static_allreduce_validation(L):
    f = L.qar_allreduce_simulated_static
    far_out = 1 << 44
    assert f(None, qar.QAR_BF16, 2, 0, 256, qar.QAR_SCHEDULE_ONE_SHOT, None, 1, None) == qar.QAR_OK   # empty call
    assert f(_arr(A, B_), qar.QAR_BF16, 2, 256, 100, 0, far_out, 1, None) == qar.QAR_ERR_UNSUPPORTED
    assert f(_arr(A, B_), qar.QAR_BF16, 2, 256, 256, 7, far_out, 1, None) == qar.QAR_ERR_UNSUPPORTED    # schedule
    assert f(_arr(A, B_), qar.QAR_BF16, 2, 256, 256, 0, far_out, 0, None) == qar.QAR_ERR_INVALID_ARG    # nchunks
    assert f(_arr(A, B_), qar.QAR_BF16, 2, 256, 256, 0, A + 64, 1, None) == qar.QAR_ERR_INVALID_ARG     # out on x
    assert f(_arr(A, B_ + 8), qar.QAR_BF16, 2, 256, 256, 0, far_out, 1, None) == qar.QAR_ERR_MISALIGNED
    # staging beyond QAR_STATIC_WORKSPACE_BYTES: one-shot over 2 ranks of 2^25 elements needs 2 x 33.6 MB
    n = 1 << 25
    assert f(_arr(A, A), qar.QAR_BF16, 2, n, 256, qar.QAR_SCHEDULE_ONE_SHOT, far_out, 1, None) == \
        qar.QAR_ERR_CAPACITY
    assert b"static workspace" in L.qar_last_error()


def test_chunked_validation(L):
    f = L.qar_reduce_quantized_chunked
    codes, scales, streams = _arr(A, B_), _arr(C, D), _arr(0x1234)
    assert f(None, None, 2, 0, 256, None, None, None, 0, 4, None, 1) == qar.QAR_OK
    assert f(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 0, streams, 1) == qar.QAR_ERR_INVALID_ARG
    assert f(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, streams, 0) == qar.QAR_ERR_INVALID_ARG
    assert f(codes, scales, 2, 256, 256, 0x50000, 0x60000, None, 0, 4, streams, 17) == qar.QAR_ERR_INVALID_ARG
    assert f(codes, scales, 2, 256, 256, 0x50000, 0x60001, None, 0, 4, streams, 1) == qar.QAR_ERR_MISALIGNED
    assert f(codes, scales, 2, 256, 256, A + 64, 0x60000, None, 0, 4, streams, 1) == qar.QAR_ERR_INVALID_ARG


def test_rows_validation(L):
    q = L.qar_quantize_rows
    assert q(A, qar.QAR_BF16, 0, 100, 256, B_, C, None) == qar.QAR_OK
    assert q(A, qar.QAR_BF16, 3, 100, 100, B_, C, None) == qar.QAR_ERR_UNSUPPORTED
    assert q(A + 1, qar.QAR_BF16, 3, 100, 256, B_, C, None) == qar.QAR_ERR_MISALIGNED   # bf16 needs 2-byte alignment
    assert q(A, qar.QAR_F32, 3, 100, 256, B_, C + 2, None) == qar.QAR_ERR_MISALIGNED
    assert q(A, qar.QAR_BF16, 3, 100, 256, A + 64, C, None) == qar.QAR_ERR_INVALID_ARG   # codes overlap x
    assert q(A, qar.QAR_BF16, 1 << 20, 1 << 21, 64, B_, C, None) == qar.QAR_ERR_INVALID_ARG   # too many elements
    # too many blocks: 2^26 rows of 100 elements, 2 blocks of 64 per row = 2^27 > QAR_MAX_ROW_BLOCKS, while
    # 6.7e9 elements stay under QAR_MAX_ELEMENTS; 100 % 64 != 0, so the flat path cannot take it.  The fake
    # ranges are disjoint (x spans 12.5 GiB from A), so the block cap is the only check that can refuse it.
    far_codes, far_scales = 1 << 44, 1 << 45
    assert q(A, qar.QAR_BF16, 1 << 26, 100, 64, far_codes, far_scales, None) == qar.QAR_ERR_INVALID_ARG
    assert q(A, qar.QAR_BF16, 1 << 25, 100, 64, far_codes, far_scales + 2, None) == qar.QAR_ERR_MISALIGNED  # at the cap
    d = L.qar_dequantize_rows
    assert d(A, C, 3, 100, 256, A + 8, qar.QAR_F32, None) == qar.QAR_ERR_INVALID_ARG        # out overlaps codes
    r = L.qar_reduce_quantized_rows
    assert r(_arr(A, B_), _arr(C, D), 2, 3, 100, 256, 0x50000, 0x60000, 0x70001, qar.QAR_BF16, None) == \
        qar.QAR_ERR_MISALIGNED
    g = L.qar_ring_step_rows
    assert g(A, C, B_, qar.QAR_BF16, 3, 100, 256, A, D, None) == qar.QAR_ERR_INVALID_ARG     # half in place


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "qar.h"

/* A plain C99 caller: argument checks return before any HIP call, so this
   runs without a GPU. */
int main(void) {
    int8_t* codes[2] = {(int8_t*)0x10000, (int8_t*)0x20000};
    float* scales[2] = {(float*)0x30000, (float*)0x40000};
    if (qar_quantize_blocks((const void*)0x10000, QAR_BF16, 0, 256, codes[0], scales[0], NULL) != QAR_OK) return 1;
    if (qar_quantize_blocks((const void*)0x10000, QAR_BF16, 256, 100, codes[0], scales[0], NULL)
        != QAR_ERR_UNSUPPORTED) return 2;
    if (qar_reduce_quantized((const int8_t* const*)codes, (const float* const*)scales, 0, 256, 256,
                             (int8_t*)0x50000, (float*)0x60000, NULL, QAR_BF16, NULL) != QAR_ERR_INVALID_ARG) return 3;
    if (qar_quantize_reduce((const void*)0x80000, QAR_BF16, 5, codes, scales, 2, 256, 256, (int8_t*)0x50000,
                            (float*)0x60000, NULL, QAR_BF16, NULL) != QAR_ERR_INVALID_ARG) return 4;
    if (qar_dequantize_e4m3((const uint8_t*)0x10001, (const float*)0x30000, 256, 256, (void*)0x80000, QAR_F32,
                            NULL) != QAR_ERR_MISALIGNED) return 5;
    if (strcmp(qar_status_string(QAR_ERR_MISALIGNED), "misaligned pointer") != 0) return 6;
    printf("%s\n", qar_status_string(QAR_OK));
    return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/qar.h compiles as C99 with warnings as errors, and a C program
    links against libqar.so and gets the documented statuses."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(qar.LIBRARY)
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(root, "include"),
                    str(src), "-o", str(exe), "-L", lib_dir, "-lqar", f"-Wl,-rpath,{lib_dir}",
                    "-Wl,-rpath-link,/opt/rocm/lib"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "ok"
