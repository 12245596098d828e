"""Pack-once / execute-many wrapper around the C entry points.

The cuDNN page ("Requirements", "Weight Packing") describes the usage this
mirrors: pack a checkpoint weight once, keep the packed copy, and execute
with preallocated buffers on the caller's stream. PyTorch only allocates
the device buffers here; every step runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (NCDHW, NDHWC, conv3d_fwd, conv3d_fwd_padded, conv3d_group_norm,
               conv3d_group_norm_workspace_bytes, conv3d_output_dims, conv3d_pack_weight,
               conv3d_pack_weight_2d, conv3d_pack_weight_fp8, conv3d_packed_weight_bytes,
               conv3d_packed_weight_bytes_fp8, conv3d_padded_workspace_bytes,
               conv3d_stream_pack_input, conv3d_workspace_bytes, make_desc, make_epilogue,
               make_group_norm_desc, make_out_pad)


def _expect(t: Optional[torch.Tensor], shape, what: str) -> None:
    """An output or operand tensor of the layer: bf16, contiguous, on a GPU,
    of exactly the layer's shape (the library sizes every access from the
    layer's descriptor)."""
    if t is None:
        return
    if (tuple(t.shape) != tuple(shape) or t.dtype != torch.bfloat16 or not t.is_contiguous()
            or not t.is_cuda):
        raise ValueError(f"{what} must be a contiguous bf16 GPU tensor of shape {tuple(shape)}, "
                         f"got {tuple(t.shape)} {t.dtype} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def pack_weight(w_oidhw: torch.Tensor, stream=None) -> torch.Tensor:
    """OIDHW bf16 [Cout][Cin][3][3][3] on the GPU -> packed weight buffer.
    A 4-D [Cout][Cin][3][3] weight is packed as the last temporal slice of a
    3x3x3 weight (for 2D and 1x3x3 layers run on single frames); an
    float8_e4m3fn 5-D weight is packed for the fp8 conv."""
    if w_oidhw.dtype == torch.float8_e4m3fn and w_oidhw.is_cuda and w_oidhw.dim() == 5:
        cout, cin = w_oidhw.shape[:2]
        w = w_oidhw.contiguous()
        out = torch.empty(conv3d_packed_weight_bytes_fp8(cout, cin), dtype=torch.uint8,
                          device=w.device)
        conv3d_pack_weight_fp8(w, out, cout, cin, stream)
        return out
    if w_oidhw.dtype != torch.bfloat16 or not w_oidhw.is_cuda or w_oidhw.dim() not in (4, 5):
        raise ValueError("weight must be a 4-D or 5-D bf16 CUDA tensor")
    cout, cin = w_oidhw.shape[:2]
    w = w_oidhw.contiguous()
    out = torch.empty(conv3d_packed_weight_bytes(cout, cin) // 2, dtype=torch.bfloat16,
                      device=w.device)
    if w.dim() == 4:
        conv3d_pack_weight_2d(w, out, cout, cin, stream)
    else:
        conv3d_pack_weight(w, out, cout, cin, stream)
    return out


class Conv3d:
    """One 3x3x3 bf16 conv layer with a packed weight and fixed shapes."""

    def __init__(self, weight: torch.Tensor, x_shape: Sequence[int], *, stride=(1, 1, 1),
                 pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), layout: int = NDHWC,
                 out_layout: Optional[int] = None, split_k: int = 0,
                 bias: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
                 norm_silu: bool = False, residual: bool = False, residual_out: bool = False,
                 out_pad_lo=None, out_pad_hi=(0, 0, 0), history_frames: int = 0,
                 cache_frames: int = 0, pad_mode: int = 0):
        """out_pad_lo / out_pad_hi: write the output into the interior of a
        zero-bordered buffer (the history_frames planes before it are the
        caller's); cache_frames > 0: also keep the last output frames in a
        cache passed to each call."""
        self.cout, self.cin = int(weight.shape[0]), int(weight.shape[1])
        self.layout = layout
        self.out_layout = layout if out_layout is None else out_layout
        self.x_shape = tuple(int(v) for v in x_shape)
        self.fp8 = weight.dtype == torch.float8_e4m3fn
        self.in_dtype = torch.float8_e4m3fn if self.fp8 else torch.bfloat16
        self.desc = make_desc(self.x_shape, self.cout, stride=stride, pad_lo=pad_lo, pad_hi=pad_hi,
                              layout=layout, out_layout=self.out_layout, split_k=split_k,
                              pad_mode=pad_mode, dtype=1 if self.fp8 else 0)
        self.out_dhw = conv3d_output_dims(self.desc)
        n = self.x_shape[0]
        if self.out_layout == NDHWC:
            self.out_shape = (n,) + self.out_dhw + (self.cout,)
        else:
            self.out_shape = (n, self.cout) + self.out_dhw
        self.padded = out_pad_lo is not None or cache_frames > 0
        self.out_pad_lo = tuple(out_pad_lo or (0, 0, 0))
        self.out_pad_hi = tuple(out_pad_hi)
        self.history_frames = history_frames
        self.cache_frames = cache_frames
        if self.padded:
            self.out_shape = (n,) + tuple(o + a + b for o, a, b in zip(
                self.out_dhw, self.out_pad_lo, self.out_pad_hi)) + (self.cout,)
            self.cache_shape = (n, cache_frames) + self.out_dhw[1:] + (self.cout,)
        self.device = weight.device
        self.w_packed = pack_weight(weight)
        self.bias = None if bias is None else bias.to(device=self.device, dtype=torch.float32).contiguous()
        self.gamma = None if gamma is None else gamma.to(device=self.device, dtype=torch.bfloat16).contiguous()
        self.norm_silu = norm_silu
        self.has_residual = residual
        self.has_residual_out = residual_out
        probe = make_epilogue(bias=self.bias, gamma=self.gamma, norm_silu=norm_silu)
        probe.flags |= (2 if residual else 0) | (8 if residual_out else 0)
        if self.padded:
            self.workspace_bytes = conv3d_padded_workspace_bytes(self.desc, probe,
                                                                 self._out_pad(None))
        else:
            self.workspace_bytes = conv3d_workspace_bytes(self.desc, probe)
        self.workspace = (torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)
                          if self.workspace_bytes else None)

    def _out_pad(self, cache):
        # the probe for the workspace size only needs a non-null cache address
        c = cache if cache is not None else (16 if self.cache_frames else None)
        return make_out_pad(self.out_pad_lo, self.out_pad_hi, self.history_frames, c,
                            self.cache_frames)

    def new_output(self) -> torch.Tensor:
        return torch.empty(self.out_shape, dtype=torch.bfloat16, device=self.device)

    def __call__(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None,
                 y: Optional[torch.Tensor] = None, residual_out: Optional[torch.Tensor] = None,
                 stream=None, cache: Optional[torch.Tensor] = None) -> torch.Tensor:
        if (tuple(x.shape) != self.x_shape or x.dtype != self.in_dtype or not x.is_contiguous()
                or not x.is_cuda):
            raise ValueError(f"x must be a contiguous {self.in_dtype} GPU tensor of shape "
                             f"{self.x_shape}")
        if self.has_residual != (residual is not None):
            raise ValueError("residual presence differs from construction")
        if self.has_residual_out != (residual_out is not None):
            raise ValueError("residual_out presence differs from construction")
        n = self.x_shape[0]
        plain = ((n,) + self.out_dhw + (self.cout,) if self.out_layout == NDHWC
                 else (n, self.cout) + self.out_dhw)
        _expect(residual, plain, "residual")
        _expect(residual_out, plain, "residual_out")
        _expect(y, self.out_shape, "y")
        if self.padded:
            _expect(cache, self.cache_shape, "cache")
        if y is None:
            y = self.new_output()
        epi = make_epilogue(bias=self.bias, residual=residual, gamma=self.gamma,
                            residual_out=residual_out, norm_silu=self.norm_silu)
        if self.padded:
            if (cache is not None) != (self.cache_frames > 0):
                raise ValueError("cache presence differs from construction")
            conv3d_fwd_padded(self.desc, x, self.w_packed, epi if epi.flags else None,
                              self._out_pad(cache), y, self.workspace, self.workspace_bytes, stream)
        else:
            conv3d_fwd(self.desc, x, self.w_packed, epi if epi.flags else None, y, self.workspace,
                       self.workspace_bytes, stream)
        return y


def stream_pack_input(chunk: torch.Tensor, history: Optional[torch.Tensor], c_pad: int,
                      padded: Optional[torch.Tensor] = None, cache: Optional[torch.Tensor] = None,
                      cache_frames: int = 2, stream=None):
    """First layer of a streaming causal encoder: chunk [N, C, T, H, W] (any
    strides) and history [N, P, H, W, C] -> (padded [N, T+2, H+2, W+2, c_pad],
    cache [N, min(cache_frames, T+P), H, W, C])."""
    n, c, t, h, w = (int(v) for v in chunk.shape)
    P = 0 if history is None else int(history.shape[1])
    cf = min(cache_frames, t + P)
    if padded is None:
        padded = torch.empty((n, t + 2, h + 2, w + 2, c_pad), dtype=torch.bfloat16,
                             device=chunk.device)
    if cache is None and cf > 0:
        cache = torch.empty((n, cf, h, w, c), dtype=torch.bfloat16, device=chunk.device)
    if history is not None:
        history = history.contiguous()
    conv3d_stream_pack_input(chunk, chunk.stride(), n, c, t, h, w, history, P, padded, c_pad,
                             cache, cf if cache is not None else 0, stream)
    return padded, cache


class GroupNorm:
    """Channels-last GroupNorm (+ SiLU) of one NDHWC activation shape, with
    its workspace allocated once; statistics per frame when t_isolated."""

    def __init__(self, x_shape: Sequence[int], groups: int, gamma: torch.Tensor,
                 beta: torch.Tensor, *, eps: float = 1e-5, silu: bool = False,
                 t_isolated: bool = True):
        self.x_shape = tuple(int(v) for v in x_shape)
        self.desc = make_group_norm_desc(self.x_shape, groups, eps=eps, silu=silu,
                                         t_isolated=t_isolated)
        self.device = gamma.device
        self.gamma = gamma.to(dtype=torch.float32).contiguous()
        self.beta = beta.to(device=self.device, dtype=torch.float32).contiguous()
        self.workspace_bytes = conv3d_group_norm_workspace_bytes(self.desc)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
        """y = GroupNorm(x); pass y=x to normalise in place."""
        if tuple(x.shape) != self.x_shape or x.dtype != torch.bfloat16 or not x.is_contiguous():
            raise ValueError(f"x must be a contiguous bf16 tensor of shape {self.x_shape}")
        if y is None:
            y = torch.empty_like(x)
        conv3d_group_norm(self.desc, x, self.gamma, self.beta, y, self.workspace,
                          self.workspace_bytes, stream)
        return y
