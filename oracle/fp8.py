"""FP8 (e4m3fn) operands for the conv oracle — TEST INFRASTRUCTURE ONLY.

The Qwen-Image PR page ("Test plan", the FP8 suite of the implicit-GEMM
conv) runs the conv with e4m3fn activations and weights, an fp32 bias and a
bf16 output. e4m3fn is 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa
bits; exponent 0 holds the subnormals m/8 * 2^-6; the pattern with all
exponent and mantissa bits set (0x7F, 0xFF) is NaN; there are no infinities,
so the largest value is 1.75 * 2^8 = 448. Every such value has at most 4
significant bits and an exponent in [-9, 8], so it is exactly a bf16 value:
the fp8 conv is the bf16 oracle conv on the decoded operands.

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this module; it shares no code with the GPU library.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(codes) -> np.ndarray:
    """e4m3fn byte codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 0xF) & (m == 0x7), np.nan, v)
    return sign * v


def e4m3_to_bf16_bits(codes) -> np.ndarray:
    """The bf16 bit patterns of e4m3fn codes (exact; NaN codes are rejected)."""
    v = e4m3_value(codes)
    if np.isnan(v).any():
        raise ValueError("NaN e4m3 code")
    f = v.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def conv3d_fp8(x_codes, w_codes, **kw):
    """Conv3D of e4m3fn x (NDHWC) and w (OIDHW) codes: the oracle conv on the
    decoded values (exact products, an fp32 accumulator, bf16 output)."""
    import oracle
    return oracle.conv3d(e4m3_to_bf16_bits(x_codes), e4m3_to_bf16_bits(w_codes), **kw)
