"""The Python binding's own checks on the CPU: it refuses host tensors,
non-contiguous tensors and unsupported dtypes before calling the library,
and turns a non-OK status into QarError with the library's text."""
import pytest
import torch

from block_wise_int8_amd import qar


def test_host_tensor_is_refused():
    x = torch.zeros(256, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="CUDA"):
        qar.qar_quantize_blocks(x, 256)
    with pytest.raises(TypeError, match="CUDA"):
        qar.qar_quantize_blocks_int4(x, 256)


def test_status_becomes_qar_error():
    with pytest.raises(qar.QarError, match="where: misaligned pointer") as e:
        qar._check(qar.QAR_ERR_MISALIGNED, "where")
    assert e.value.status == qar.QAR_ERR_MISALIGNED
    with pytest.raises(qar.QarError, match="unsupported block size or dtype"):
        qar._check(qar.QAR_ERR_UNSUPPORTED, "x")
    qar._check(qar.QAR_OK, "fine")


def test_dtypes():
    assert qar._dtype_code(torch.bfloat16) == qar.QAR_BF16
    assert qar._dtype_code(torch.float32) == qar.QAR_F32
    with pytest.raises(TypeError, match="bfloat16 and float32"):
        qar._dtype_code(torch.float16)


class _AsCuda(torch.Tensor):
    """A host tensor that reports itself as a device tensor, so that the
    contiguity check is the one that refuses it (no GPU is touched)."""
    @property
    def is_cuda(self):
        return True


def test_non_contiguous_is_refused():
    t = torch.zeros(4, 4).t().as_subclass(_AsCuda)
    assert t.is_cuda and not t.is_contiguous()
    with pytest.raises(ValueError, match="codes must be contiguous"):
        qar._dev(t, "codes")


# ---------------------------------------------------------------------------
# size, dtype and device checks: the C ABI sees only pointers, so the binding
# refuses any tensor that does not fit the call before the library is called
# (every case below raises in Python; no pointer reaches libqar).


def _d(n, dtype, device="cpu"):
    return torch.zeros(n, dtype=dtype, device=device).as_subclass(_AsCuda)


N_ = 1024
B_ = 256


def _ranks(k=3, n=N_, codes_dtype=torch.int8):
    return [_d(n, codes_dtype) for _ in range(k)], [_d(n // B_, torch.float32) for _ in range(k)]


def test_quantize_refuses_ill_fitting_outputs():
    x = _d(N_, torch.bfloat16)
    with pytest.raises(ValueError, match="codes must hold 1024"):
        qar.qar_quantize_blocks(x, B_, codes=_d(N_ - 16, torch.int8), scales=_d(4, torch.float32))
    with pytest.raises(TypeError, match="codes must be"):
        qar.qar_quantize_blocks(x, B_, codes=_d(N_, torch.float32), scales=_d(4, torch.float32))
    with pytest.raises(TypeError, match="scales must be torch.float32"):
        qar.qar_quantize_blocks(x, B_, codes=_d(N_, torch.int8), scales=_d(4, torch.bfloat16))
    with pytest.raises(ValueError, match="scales must hold 4"):
        qar.qar_quantize_blocks(x, B_, codes=_d(N_, torch.int8), scales=_d(3, torch.float32))
    with pytest.raises(ValueError, match="codes must hold 512"):        # 4-bit: n/2 bytes
        qar.qar_quantize_blocks_int4(x, B_, codes=_d(N_, torch.uint8), scales=_d(4, torch.float32))


def test_reduce_refuses_ill_fitting_ranks_and_outputs():
    codes, scales = _ranks()
    short = [codes[0], _d(N_ - 16, torch.int8), codes[2]]
    with pytest.raises(ValueError, match=r"codes\[1\] must hold 1024"):
        qar.qar_reduce_quantized(short, scales, B_, _d(N_, torch.int8), _d(4, torch.float32))
    bad_s = [scales[0], scales[1], _d(4, torch.bfloat16)]
    with pytest.raises(TypeError, match=r"scales\[2\] must be torch.float32"):
        qar.qar_reduce_quantized(codes, bad_s, B_, _d(N_, torch.int8), _d(4, torch.float32))
    with pytest.raises(ValueError, match="codes_out must hold 1024"):
        qar.qar_reduce_quantized(codes, scales, B_, _d(N_ - 1, torch.int8), _d(4, torch.float32))
    with pytest.raises(ValueError, match="scales_out must hold 4"):
        qar.qar_reduce_quantized(codes, scales, B_, _d(N_, torch.int8), _d(2, torch.float32))
    with pytest.raises(ValueError, match="out must hold 1024"):
        qar.qar_reduce_quantized(codes, scales, B_, _d(N_, torch.int8), _d(4, torch.float32),
                                 out=_d(N_ - 1, torch.bfloat16))
    with pytest.raises(TypeError, match="out must be"):
        qar.qar_reduce_quantized(codes, scales, B_, _d(N_, torch.int8), _d(4, torch.float32),
                                 out=_d(N_, torch.int16))
    other = [codes[0], codes[1], _d(N_, torch.int8, "meta")]
    with pytest.raises(ValueError, match=r"codes\[2\] is on meta"):
        qar.qar_reduce_quantized(other, scales, B_, _d(N_, torch.int8), _d(4, torch.float32))
    c4, s4 = _ranks(codes_dtype=torch.uint8)
    with pytest.raises(ValueError, match=r"codes\[1\] must hold 1024"):   # n = 2048 elements of 4-bit codes
        qar.qar_reduce_quantized_int4([c4[0], _d(N_ // 2, torch.uint8)], [_d(8, torch.float32)] * 2, B_)
    with pytest.raises(ValueError, match=r"codes\[1\] must hold 1024"):
        qar.qar_reduce_quantized_pipelined([codes[0], codes[1][:-16].as_subclass(_AsCuda)], scales[:2], B_, 4,
                                           [None], _d(N_, torch.int8), _d(4, torch.float32))


def test_quantize_reduce_and_ring_refuse_ill_fitting_tensors():
    codes, scales = _ranks()
    x = _d(N_, torch.bfloat16)
    with pytest.raises(ValueError, match=r"codes\[2\] must hold 1024"):
        qar.qar_quantize_reduce(x, 0, [codes[0], codes[1], _d(512, torch.int8)], scales, B_)
    with pytest.raises(ValueError, match=r"scales\[0\] must hold 4"):
        qar.qar_quantize_reduce(x, 0, codes, [_d(8, torch.float32), scales[1], scales[2]], B_)
    with pytest.raises(ValueError, match="codes_in must hold 1024"):
        qar.qar_ring_step(_d(N_ // 2, torch.int8), scales[0], x, B_)
    with pytest.raises(ValueError, match="scales_in must hold 4"):
        qar.qar_ring_step(codes[0], _d(1, torch.float32), x, B_)
    with pytest.raises(ValueError, match="codes_out must hold 1024"):
        qar.qar_ring_step(codes[0], scales[0], x, B_, codes_out=_d(N_ // 2, torch.int8))


def test_dequantize_refuses_ill_fitting_tensors():
    with pytest.raises(ValueError, match="scales must hold 4"):
        qar.qar_dequantize(_d(N_, torch.int8), _d(2, torch.float32), B_)
    with pytest.raises(ValueError, match="out must hold 1024"):
        qar.qar_dequantize(_d(N_, torch.int8), _d(4, torch.float32), B_, out=_d(N_ - 8, torch.float32))
    with pytest.raises(TypeError, match="codes must be"):
        qar.qar_dequantize(_d(N_, torch.float32), _d(4, torch.float32), B_)
    with pytest.raises(ValueError, match="scales must hold 4"):          # 4-bit: 512 bytes hold 1024 elements
        qar.qar_dequantize_int4(_d(N_ // 2, torch.uint8), _d(2, torch.float32), B_)


def test_comparator_and_simulated_allreduce_refuse_ill_fitting_tensors():
    xs = [_d(N_, torch.bfloat16) for _ in range(3)]
    with pytest.raises(ValueError, match=r"x\[1\] must hold 1024"):
        qar.qar_reduce_unquantized([xs[0], _d(N_ - 16, torch.bfloat16)])
    with pytest.raises(TypeError, match=r"x\[1\] must be torch.bfloat16"):
        qar.qar_reduce_unquantized([xs[0], _d(N_, torch.float32)])
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        qar.qar_reduce_unquantized(xs, out=_d(N_, torch.float32))
    wc, ws = _ranks()
    with pytest.raises(ValueError, match="needs 3 codes and scales workspaces"):
        qar.qar_allreduce_simulated(xs, B_, "one_shot", out=_d(N_, torch.bfloat16), workspace=(wc[:2], ws[:2]),
                                    streams=[None])
    with pytest.raises(ValueError, match=r"workspace codes\[1\] must hold 1024"):
        qar.qar_allreduce_simulated(xs, B_, "one_shot", out=_d(N_, torch.bfloat16),
                                    workspace=([wc[0], _d(16, torch.int8), wc[2]], ws), streams=[None])
    with pytest.raises(ValueError, match=r"workspace scales\[0\] must hold 4"):
        qar.qar_allreduce_simulated(xs, B_, "ring", out=_d(N_, torch.bfloat16),
                                    workspace=([wc[0]], [_d(1, torch.float32)]), streams=[None])
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        qar.qar_allreduce_simulated(xs, B_, "ring", out=_d(N_, torch.float32), workspace=(wc, ws), streams=[None])


def test_rows_calls_refuse_ill_fitting_tensors():
    rows, row_len, block = 4, 300, 256                     # 2 blocks per row (one partial)
    x = torch.zeros(rows, row_len, dtype=torch.bfloat16).as_subclass(_AsCuda)
    with pytest.raises(ValueError, match="codes must hold 1200"):
        qar.qar_quantize_rows(x, block, codes=_d(1100, torch.int8))
    with pytest.raises(ValueError, match="scales must hold 8"):
        qar.qar_quantize_rows(x, block, codes=_d(1200, torch.int8), scales=_d(4, torch.float32))
    codes, scales = [_d(1200, torch.int8)] * 2, [_d(8, torch.float32)] * 2
    with pytest.raises(ValueError, match=r"scales\[1\] must hold 8"):
        qar.qar_reduce_quantized_rows(codes, [scales[0], _d(7, torch.float32)], rows, row_len, block)
    with pytest.raises(ValueError, match="out must hold 1200"):
        qar.qar_reduce_quantized_rows(codes, scales, rows, row_len, block, _d(1200, torch.int8),
                                      _d(8, torch.float32), out=_d(1000, torch.bfloat16))
    with pytest.raises(ValueError, match="codes_in must hold 1200"):
        qar.qar_ring_step_rows(_d(1000, torch.int8), scales[0], x, block)
    with pytest.raises(ValueError, match="scales must hold 8"):
        qar.qar_dequantize_rows(codes[0], _d(6, torch.float32), rows, row_len, block)
