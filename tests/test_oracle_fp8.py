"""Pins for the e4m3fn decoding the fp8 conv oracle rests on: PyTorch's own
float8_e4m3fn conversion (a library cast) over all 256 codes, hand-decoded
codes from the format definition, exactness in bf16, and one fp8 conv
against a conv of the same decoded values computed by F.conv3d in fp64."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.fp8 import conv3d_fp8, e4m3_to_bf16_bits, e4m3_value


def test_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_value(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0xB8, -1.0), (0x40, 2.0), (0x7E, 448.0),
                                        (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                        (0x3C, 1.5), (0x00, 0.0), (0x80, -0.0)])
def test_hand_decoded_codes(code, value):
    assert e4m3_value([code])[0] == value
    assert np.signbit(e4m3_value([code])[0]) == np.signbit(value)


def test_every_finite_code_is_exact_in_bf16():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    bits = e4m3_to_bf16_bits(codes)
    assert np.array_equal(oracle.bf16_to_f32(bits).astype(np.float64), e4m3_value(codes))
    with pytest.raises(ValueError):
        e4m3_to_bf16_bits([0x7F])


def test_fp8_conv_matches_fp64_conv_of_decoded_values():
    rng = np.random.default_rng(61)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    x = rng.choice(finite, size=(1, 4, 5, 6, 16))
    w = rng.choice(finite[np.abs(e4m3_value(finite)) < 2], size=(32, 16, 3, 3, 3))
    got = conv3d_fp8(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    xt = torch.from_numpy(e4m3_value(x)).permute(0, 4, 1, 2, 3)
    xt = F.pad(xt, (1, 1, 1, 1, 2, 0))
    ref = F.conv3d(xt, torch.from_numpy(e4m3_value(w))).permute(0, 2, 3, 4, 1).numpy()
    assert np.array_equal(got["acc"].astype(np.float64), ref.astype(np.float32).astype(np.float64))
