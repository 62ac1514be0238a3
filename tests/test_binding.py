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
