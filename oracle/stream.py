"""Streaming causal conv oracle: padded outputs, history planes, caches and
the standalone post-operations — TEST INFRASTRUCTURE ONLY.

What it computes. The cuDNN frontend page "Fused Conv3D + Bias + Residual +
RMSNorm + SiLU" describes how a video VAE runs its causal convs on temporal
chunks ("Causal Conv3D with Cache", "Normalization and Padding Variant",
"Spatial Padding Variant"): a layer writes its activations into the interior
of a larger buffer whose border is zero and whose two leading temporal planes
hold the previous chunk's last two activated frames (its "history"), and it
keeps those last frames in a small cache for the next chunk. The next conv
then runs as a valid conv on that buffer: the history planes stand where the
causal zero planes would be, the zero border is the spatial padding. The
first layer packs its raw input chunk (channels-first, 12 channels in the
page's workload) the same way, with zero channels up to a multiple of 8.

Everything here is data movement on bf16 bit patterns (uint16 arrays), so it
is exact. The convolutions are oracle.conv3d's.

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this module; it shares no code with the GPU library.
"""
from __future__ import annotations

import numpy as np


def pad_output(y, pad_lo, pad_hi, history=None):
    """y [N, D, H, W, C] -> [N, D+pt+qt, H+ph+qh, W+pw+qw, C] with y in the
    interior and zeros elsewhere, except that with history [N, P, H, W, C]
    (P <= pt) the interiors of planes pt-P .. pt-1 hold the history."""
    y = np.asarray(y)
    N, D, H, W, C = y.shape
    (pt, ph, pw), (qt, qh, qw) = pad_lo, pad_hi
    out = np.zeros((N, D + pt + qt, H + ph + qh, W + pw + qw, C), dtype=y.dtype)
    out[:, pt:pt + D, ph:ph + H, pw:pw + W] = y
    if history is not None and history.shape[1]:
        P = history.shape[1]
        if P > pt:
            raise ValueError("more history frames than leading planes")
        out[:, pt - P:pt, ph:ph + H, pw:pw + W] = history
    return out


def cache_tail(current, cache_frames, previous=None):
    """The last cache_frames frames of previous ++ current (along D)."""
    frames = current if previous is None else np.concatenate([previous, current], axis=1)
    if cache_frames > frames.shape[1]:
        raise ValueError("cache longer than the frames seen")
    return frames[:, frames.shape[1] - cache_frames:].copy()


def pack_stream_input(chunk_ncthw, history=None, c_pad=16):
    """First layer of a streaming causal encoder: a channels-first chunk
    [N, C, T, H, W] and up to two raw history frames [N, P, H, W, C] (NDHWC)
    -> (padded [N, T+2, H+2, W+2, c_pad], cache [N, min(2, T+P), H, W, C]).

    padded holds the chunk (channels-last) in planes 2 .. T+1, the history in
    the P planes before them, zeros in the 2-P missing-history planes, the
    one-pixel spatial border and channels C .. c_pad-1; cache holds the last
    raw frames of history ++ chunk."""
    x = np.ascontiguousarray(np.transpose(np.asarray(chunk_ncthw), (0, 2, 3, 4, 1)))
    N, T, H, W, C = x.shape
    if c_pad < C:
        raise ValueError("c_pad below the channel count")
    P = 0 if history is None else history.shape[1]
    if P > 2:
        raise ValueError("at most two history frames")
    xc = np.zeros((N, T, H, W, c_pad), dtype=x.dtype)
    xc[..., :C] = x
    hc = None
    if P:
        hc = np.zeros((N, P, H, W, c_pad), dtype=x.dtype)
        hc[..., :C] = history
    padded = pad_output(xc, (2, 1, 1), (0, 1, 1), history=hc)
    cache = cache_tail(x, min(2, T + P), previous=history if P else None)
    return padded, cache


def _b(v):
    """B(): fp32 -> bf16 (nearest, ties to even) -> fp32."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = v.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32)


def _bits(v):
    """bf16 bit patterns of fp32 values that are already bf16."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def norm_silu(raw, gamma, *, bias=None, residual=None, intermediates=False):
    """The cuDNN page's post-operations ("Operation Contract") applied to an
    existing bf16 tensor raw [..., C] (a raw conv output: conv = raw), as the
    page's standalone normalization variant ("Standalone Normalization and
    Padding Variant") does for channel counts above the fused tile:

      main  = B(conv + bias)            (bias fp32 [C], optional)
      value = B(main + residual)        (residual bf16, optional)
      den   = max(sqrt(sum_c value^2), 1e-12)
      y     = B(a / (1 + exp(-a))),  a = B(B(B(value / den) * sqrt(C)) * gamma)

    fp32 arithmetic (IEEE, correctly rounded), the sum of squares in float64
    rounded once to fp32, exp in float64 rounded once to fp32. Returns y bits,
    or with intermediates a dict of y, conv, main, value, affine (bits) and
    den (fp32)."""
    conv = (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    C = conv.shape[-1]
    main = _b(conv + np.asarray(bias, dtype=np.float32)) if bias is not None else conv
    value = main
    if residual is not None:
        res = (np.asarray(residual, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        value = _b(main + res)
    ss = np.sum(value.astype(np.float64) ** 2, axis=-1, keepdims=True)
    den = np.maximum(np.sqrt(ss.astype(np.float32)), np.float32(1e-12))
    g = (np.asarray(gamma, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    nrm = _b(value / den)
    scl = _b(nrm * np.sqrt(np.float32(C)))
    aff = _b(scl * g)
    e = np.exp(-aff.astype(np.float64)).astype(np.float32)
    y = _bits(_b(aff / (np.float32(1.0) + e)))
    if not intermediates:
        return y
    return {"y": y, "conv": _bits(conv), "main": _bits(main), "value": _bits(value),
            "affine": _bits(aff), "den": den[..., 0].astype(np.float32)}
