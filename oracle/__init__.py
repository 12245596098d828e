"""Conv3D, GroupNorm and streaming oracle — TEST INFRASTRUCTURE ONLY.

A plain CPU direct convolution (C, OpenMP) with the cuDNN page's
"Operation Contract" post-operations (zero or reflect spatial padding), a plain channels-last GroupNorm
(+ SiLU, numpy float64, in groupnorm.py) and the streaming scheme's padded
outputs, history planes and caches (numpy, in stream.py), used to check the
GPU library.
Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package. It shares no code with the GPU library; both sides see
the same seeded inputs and nothing else.

Arrays of bf16 values are passed as numpy uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_conv3d_oracle.so")
_lib = None

BIAS = 1
RESIDUAL = 2
NORM_SILU = 4


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_SO)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_conv3d.restype = i
        lib.oracle_conv3d.argtypes = [p, p] + [i] * 9 + [p, p, p, p, p, p, i, p, ctypes.c_int64] + [p] * 7
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [ctypes.c_float]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_output_dims.restype = i
        lib.oracle_output_dims.argtypes = [i] * 6 + [p, p, p, p]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i3(v):
    return np.ascontiguousarray(np.asarray(v, dtype=np.int32).reshape(3))


def bf16_round(values) -> np.ndarray:
    """B(x) for each fp32 value: the oracle's own round-to-nearest-even."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_bf16_round(float(f)) for f in v], dtype=np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def output_dims(in_dhw, kernel, stride, pad_lo, pad_hi):
    lib = _load()
    out = np.zeros(3, dtype=np.int32)
    st = _i3(stride); lo = _i3(pad_lo); hi = _i3(pad_hi)
    rc = lib.oracle_output_dims(int(in_dhw[0]), int(in_dhw[1]), int(in_dhw[2]),
                                int(kernel[0]), int(kernel[1]), int(kernel[2]),
                                _ptr(st), _ptr(lo), _ptr(hi), _ptr(out))
    return tuple(int(v) for v in out), rc == 0


def conv3d(x, w, *, stride=(1, 1, 1), pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), bias=None,
           residual=None, gamma=None, norm_silu=False, pixels=None, intermediates=False):
    """Direct Conv3D of x (NDHWC bf16 bits) with w (OIDHW bf16 bits).

    bias: fp32 [Co]; residual: bf16 bits shaped like the NDHWC output;
    gamma: bf16 bits [Co] (required with norm_silu).
    pixels: optional flat output-pixel indices; the result is then [len, Co].
    Returns the bf16 output bits (NDHWC, or [len, Co] with pixels) or, with
    intermediates=True, a dict holding y, acc, conv, main, value, affine, den.
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    N, D, H, W, Ci = x.shape
    Co, Ci2, KD, KH, KW = w.shape
    if Ci2 != Ci:
        raise ValueError("channel mismatch")
    (Do, Ho, Wo), ok = output_dims((D, H, W), (KD, KH, KW), stride, pad_lo, pad_hi)
    if not ok:
        raise ValueError("empty output")
    M = N * Do * Ho * Wo
    flags = 0
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(Co)
        flags |= BIAS
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16).reshape(M, Co)
        flags |= RESIDUAL
    if norm_silu:
        if gamma is None:
            raise ValueError("norm_silu needs gamma")
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16).reshape(Co)
        flags |= NORM_SILU
    if pixels is not None:
        pix = np.ascontiguousarray(pixels, dtype=np.int64).ravel()
        if pix.size and (pix.min() < 0 or pix.max() >= M):
            raise ValueError("pixel index out of range")
        npix = pix.size
    else:
        pix = None
        npix = M
    y = np.empty((npix, Co), dtype=np.uint16)
    extra = {}
    if intermediates:
        extra = dict(acc=np.empty((npix, Co), np.float32), conv=np.empty((npix, Co), np.uint16),
                     main=np.empty((npix, Co), np.uint16), value=np.empty((npix, Co), np.uint16),
                     affine=np.zeros((npix, Co), np.uint16), den=np.zeros((npix,), np.float32))
    st = _i3(stride); lo = _i3(pad_lo); hi = _i3(pad_hi)
    rc = lib.oracle_conv3d(_ptr(x), _ptr(w), N, D, H, W, Ci, Co, KD, KH, KW,
                           _ptr(st), _ptr(lo), _ptr(hi), _ptr(bias), _ptr(residual),
                           _ptr(gamma), flags, _ptr(pix), npix, _ptr(y),
                           _ptr(extra.get("acc")), _ptr(extra.get("conv")),
                           _ptr(extra.get("main")), _ptr(extra.get("value")),
                           _ptr(extra.get("affine")), _ptr(extra.get("den")))
    if rc != 0:
        raise RuntimeError(f"oracle_conv3d failed ({rc})")
    shape = (N, Do, Ho, Wo, Co) if pixels is None else (npix, Co)
    if not intermediates:
        return y.reshape(shape)
    out = {k: (v.reshape(shape) if v.ndim == 2 else v) for k, v in extra.items()}
    out["y"] = y.reshape(shape)
    return out


def group_norm(x, groups, gamma, beta, **kw):
    """Channels-last GroupNorm (+ SiLU); see oracle/groupnorm.py."""
    from .groupnorm import group_norm as _gn
    return _gn(x, groups, gamma, beta, **kw)


def reflect_pad_hw(x, pad_lo, pad_hi):
    """Reflect padding of H and W of an NDHWC array (the border row or column
    itself is not repeated: index -k maps to k, H-1+k to H-1-k), as the H3
    encoder pads spatially before each conv (FlyDSL issue, H3 comment, the
    conv call site). pad_lo / pad_hi: (h, w) amounts, each < the extent."""
    x = np.asarray(x)
    (ph, pw), (qh, qw) = pad_lo, pad_hi
    H, W = x.shape[2], x.shape[3]
    if max(ph, qh) >= H or max(pw, qw) >= W:
        raise ValueError("reflect padding must be smaller than the extent")
    rows = [abs(i) if i < 0 else (2 * (H - 1) - i if i >= H else i) for i in range(-ph, H + qh)]
    cols = [abs(j) if j < 0 else (2 * (W - 1) - j if j >= W else j) for j in range(-pw, W + qw)]
    return x[:, :, rows][:, :, :, cols]


def conv3d_reflect(x, w, *, stride=(1, 1, 1), pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), **kw):
    """conv3d with zero padding in time and reflect padding in H and W: the
    input reflect-padded first, then the conv with the temporal pad only."""
    xp = reflect_pad_hw(x, pad_lo[1:], pad_hi[1:])
    return conv3d(xp, w, stride=stride, pad_lo=(pad_lo[0], 0, 0), pad_hi=(pad_hi[0], 0, 0), **kw)
