"""Host-side argument checks of the Python binding and the layer wrapper.

The library sizes every device access from the descriptor, so a tensor that
is too small, of another dtype, strided or on the host must be refused before
the C call. These checks run on the CPU: they use stand-in objects with the
tensor attributes the checks read, and never reach the library's launches.
"""
import pytest
import torch

import convolution_video_vae_amd as cv
from convolution_video_vae_amd import layer


class FakeGpuTensor:
    """The attributes _check_buffer reads, for a GPU tensor that does not exist."""

    def __init__(self, numel, dtype=torch.bfloat16, contiguous=True, cuda=True):
        self._n, self.dtype, self._c, self.is_cuda = numel, dtype, contiguous, cuda

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return 1 << 20      # never dereferenced: no test here reaches the library


def test_buffer_check_accepts_exact_and_larger():
    cv._check_buffer(FakeGpuTensor(100), 200, "y", "bf16")
    cv._check_buffer(FakeGpuTensor(101), 200, "y", "bf16")
    cv._check_buffer(None, 200, "y")
    cv._check_buffer(12345, 200, "y")        # a raw address is the caller's


@pytest.mark.parametrize("t,msg", [
    (FakeGpuTensor(99), "holds 198 bytes"),
    (FakeGpuTensor(100, dtype=torch.float32), "must be bf16"),
    (FakeGpuTensor(100, contiguous=False), "contiguous"),
    (FakeGpuTensor(100, cuda=False), "GPU tensor"),
])
def test_buffer_check_rejects(t, msg):
    with pytest.raises(ValueError, match=msg):
        cv._check_buffer(t, 200, "y", "bf16")


def test_conv_buffers_sized_from_the_descriptor():
    d = cv.make_desc((1, 5, 16, 16, 64), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    out = 1 * 5 * 16 * 16 * 128
    x = FakeGpuTensor(5 * 16 * 16 * 64)
    wp = FakeGpuTensor(cv.conv3d_packed_weight_bytes(128, 64) // 2)
    cv._check_conv_buffers(d, x, wp, None, FakeGpuTensor(out))
    with pytest.raises(ValueError, match="y holds"):
        cv._check_conv_buffers(d, x, wp, None, FakeGpuTensor(out - 8))
    with pytest.raises(ValueError, match="x holds"):
        cv._check_conv_buffers(d, FakeGpuTensor(5 * 16 * 16 * 64 - 1), wp, None, FakeGpuTensor(out))
    with pytest.raises(ValueError, match="w_packed holds"):
        cv._check_conv_buffers(d, x, FakeGpuTensor(100), None, FakeGpuTensor(out))
    epi = cv.make_epilogue(bias=FakeGpuTensor(128, dtype=torch.float32),
                           residual=FakeGpuTensor(out - 1))
    with pytest.raises(ValueError, match="residual holds"):
        cv._check_conv_buffers(d, x, wp, epi, FakeGpuTensor(out))
    epi = cv.make_epilogue(bias=FakeGpuTensor(128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bias must be fp32"):
        cv._check_conv_buffers(d, x, wp, epi, FakeGpuTensor(out))
    epi = cv.make_epilogue(gamma=FakeGpuTensor(127), norm_silu=True)
    with pytest.raises(ValueError, match="gamma holds"):
        cv._check_conv_buffers(d, x, wp, epi, FakeGpuTensor(out))
    epi = cv.make_epilogue(residual=FakeGpuTensor(out), residual_out=FakeGpuTensor(out // 2))
    with pytest.raises(ValueError, match="residual_out holds"):
        cv._check_conv_buffers(d, x, wp, epi, FakeGpuTensor(out))


def test_layer_expect_rejects_wrong_tensors():
    shape = (1, 5, 16, 16, 64)
    layer._expect(None, shape, "y")
    with pytest.raises(ValueError, match="shape"):
        layer._expect(torch.empty((1, 5, 16, 16, 32), dtype=torch.bfloat16), shape, "y")
    with pytest.raises(ValueError, match="bf16"):
        layer._expect(torch.empty(shape, dtype=torch.float32), shape, "residual")
    t = torch.empty((1, 5, 16, 64, 16), dtype=torch.bfloat16).transpose(3, 4)
    with pytest.raises(ValueError, match="not contiguous"):
        layer._expect(t, shape, "cache")
    # right shape and dtype, but a host tensor
    with pytest.raises(ValueError, match="GPU"):
        layer._expect(torch.empty(shape, dtype=torch.bfloat16), shape, "residual_out")
