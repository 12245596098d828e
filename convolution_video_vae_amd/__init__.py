"""Python binding of the MI355X Conv3D library (libconv3d_mi355x.so).

Argument marshalling only: every function below forwards to the C entry
point of the same name in include/conv3d.h, passing device pointers of
PyTorch tensors and the current HIP stream. PyTorch supplies device memory
and streams; all computation runs in the library's HIP kernels. There is no
fallback: if the shared library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONV3D_LIB selects another build of the same library (A/B timing).
LIB_PATH = os.environ.get("CONV3D_LIB") or os.path.join(_HERE, "libconv3d_mi355x.so")

NCDHW = 0
NDHWC = 1

PAD_ZERO = 0
PAD_REFLECT = 1

BF16 = 0
FP8_E4M3 = 1

EPI_BIAS = 1
EPI_RESIDUAL = 2
EPI_L2NORM_SILU = 4
EPI_RESIDUAL_OUT = 8

STATUS = {0: "CONV3D_OK", 1: "CONV3D_ERR_NULL", 2: "CONV3D_ERR_SHAPE", 3: "CONV3D_ERR_ALIGN",
          4: "CONV3D_ERR_OVERLAP", 5: "CONV3D_ERR_WORKSPACE", 6: "CONV3D_ERR_UNSUPPORTED",
          7: "CONV3D_ERR_HIP"}

EXPORTED = ("conv3d_packed_weight_bytes", "conv3d_pack_weight", "conv3d_output_dims",
            "conv3d_workspace_bytes", "conv3d_fwd", "conv3d_transpose", "conv3d_status_str",
            "conv3d_plan_describe", "conv3d_group_norm_workspace_bytes", "conv3d_group_norm",
            "conv3d_padded_workspace_bytes", "conv3d_fwd_padded", "conv3d_stream_pack_input",
            "conv3d_pack_weight_2d", "conv3d_norm_silu", "conv3d_packed_weight_bytes_fp8",
            "conv3d_pack_weight_fp8", "conv3d_fwd_noalloc", "conv3d_gn_partials_bytes",
            "conv3d_fwd_gn_stats", "conv3d_group_norm_from_partials")


class Conv3dError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_str(status)})")


class conv3d_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("d", ctypes.c_int), ("h", ctypes.c_int), ("w", ctypes.c_int),
                ("cin", ctypes.c_int), ("cout", ctypes.c_int),
                ("stride", ctypes.c_int * 3), ("pad_lo", ctypes.c_int * 3),
                ("pad_hi", ctypes.c_int * 3), ("layout", ctypes.c_int),
                ("out_layout", ctypes.c_int), ("split_k", ctypes.c_int),
                ("pad_mode", ctypes.c_int), ("dtype", ctypes.c_int)]


class conv3d_epilogue(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint), ("bias", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("residual_out", ctypes.c_void_p)]


class conv3d_out_pad(ctypes.Structure):
    _fields_ = [("pad_lo", ctypes.c_int * 3), ("pad_hi", ctypes.c_int * 3),
                ("history_frames", ctypes.c_int), ("cache_frames", ctypes.c_int),
                ("cache", ctypes.c_void_p)]


class conv3d_group_norm_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("d", ctypes.c_int), ("h", ctypes.c_int), ("w", ctypes.c_int),
                ("c", ctypes.c_int), ("groups", ctypes.c_int), ("t_isolated", ctypes.c_int),
                ("silu", ctypes.c_int), ("eps", ctypes.c_float)]


_lib = None


def lib():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python convolution_video_vae_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        pd, pe = ctypes.POINTER(conv3d_desc), ctypes.POINTER(conv3d_epilogue)
        L.conv3d_packed_weight_bytes.restype = sz
        L.conv3d_packed_weight_bytes.argtypes = [i, i]
        L.conv3d_pack_weight.restype = i
        L.conv3d_pack_weight.argtypes = [vp, vp, i, i, vp]
        L.conv3d_packed_weight_bytes_fp8.restype = sz
        L.conv3d_packed_weight_bytes_fp8.argtypes = [i, i]
        L.conv3d_pack_weight_fp8.restype = i
        L.conv3d_pack_weight_fp8.argtypes = [vp, vp, i, i, vp]
        L.conv3d_pack_weight_2d.restype = i
        L.conv3d_pack_weight_2d.argtypes = [vp, vp, i, i, vp]
        L.conv3d_output_dims.restype = i
        L.conv3d_output_dims.argtypes = [pd, ctypes.POINTER(ctypes.c_int * 3)]
        L.conv3d_workspace_bytes.restype = i
        L.conv3d_workspace_bytes.argtypes = [pd, pe, ctypes.POINTER(sz)]
        L.conv3d_fwd.restype = i
        L.conv3d_fwd.argtypes = [pd, vp, vp, pe, vp, vp, sz, vp]
        L.conv3d_fwd_noalloc.restype = i
        L.conv3d_fwd_noalloc.argtypes = [pd, vp, vp, pe, vp, vp]
        L.conv3d_transpose.restype = i
        L.conv3d_transpose.argtypes = [vp, i, vp, i, i, i, i, i, vp]
        L.conv3d_status_str.restype = ctypes.c_char_p
        L.conv3d_status_str.argtypes = [i]
        L.conv3d_plan_describe.restype = i
        L.conv3d_plan_describe.argtypes = [pd, pe, ctypes.c_char_p, sz]
        po = ctypes.POINTER(conv3d_out_pad)
        L.conv3d_padded_workspace_bytes.restype = i
        L.conv3d_padded_workspace_bytes.argtypes = [pd, pe, po, ctypes.POINTER(sz)]
        L.conv3d_fwd_padded.restype = i
        L.conv3d_fwd_padded.argtypes = [pd, vp, vp, pe, po, vp, vp, sz, vp]
        L.conv3d_stream_pack_input.restype = i
        L.conv3d_stream_pack_input.argtypes = [vp, ctypes.POINTER(ctypes.c_longlong * 5), i, i, i, i,
                                               i, vp, i, vp, i, vp, i, vp]
        L.conv3d_norm_silu.restype = i
        L.conv3d_norm_silu.argtypes = [vp, i, i, i, i, i, pe, po, vp, vp, vp]
        pg = ctypes.POINTER(conv3d_group_norm_desc)
        L.conv3d_group_norm_workspace_bytes.restype = i
        L.conv3d_group_norm_workspace_bytes.argtypes = [pg, ctypes.POINTER(sz)]
        L.conv3d_group_norm.restype = i
        L.conv3d_group_norm.argtypes = [pg, vp, vp, vp, vp, vp, sz, vp]
        L.conv3d_gn_partials_bytes.restype = i
        L.conv3d_gn_partials_bytes.argtypes = [pd, ctypes.POINTER(sz)]
        L.conv3d_fwd_gn_stats.restype = i
        L.conv3d_fwd_gn_stats.argtypes = [pd, vp, vp, vp, vp, vp, sz, vp]
        L.conv3d_group_norm_from_partials.restype = i
        L.conv3d_group_norm_from_partials.argtypes = [pg, pd, vp, vp, vp, vp, vp, vp, sz, vp]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().conv3d_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise Conv3dError(status, what)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_desc(x_shape: Sequence[int], cout: int, *, stride=(1, 1, 1), pad_lo=(0, 0, 0),
              pad_hi=(0, 0, 0), layout=NDHWC, out_layout=None, split_k=0,
              pad_mode=PAD_ZERO, dtype=BF16) -> conv3d_desc:
    """Descriptor from the input shape in `layout` (NDHWC or NCDHW)."""
    if layout == NDHWC:
        n, d, h, w, cin = x_shape
    else:
        n, cin, d, h, w = x_shape
    return conv3d_desc(n, d, h, w, cin, cout, (ctypes.c_int * 3)(*stride),
                       (ctypes.c_int * 3)(*pad_lo), (ctypes.c_int * 3)(*pad_hi), layout,
                       layout if out_layout is None else out_layout, split_k, pad_mode, dtype)


def make_epilogue(bias=None, residual=None, gamma=None, residual_out=None,
                  norm_silu=False) -> conv3d_epilogue:
    flags = 0
    flags |= EPI_BIAS if bias is not None else 0
    flags |= EPI_RESIDUAL if residual is not None else 0
    flags |= EPI_L2NORM_SILU if norm_silu else 0
    flags |= EPI_RESIDUAL_OUT if residual_out is not None else 0
    e = conv3d_epilogue(flags, _ptr(bias), _ptr(residual), _ptr(gamma), _ptr(residual_out))
    # the tensors themselves, so the calls can check their sizes and types
    e.tensors = dict(bias=bias, residual=residual, gamma=gamma, residual_out=residual_out)
    return e


_DTYPE_NAMES = {"bf16": "bfloat16", "fp32": "float32"}


def _check_buffer(t, nbytes: int, what: str, dtype: Optional[str] = None) -> None:
    """A tensor handed to the library as a buffer must be a contiguous GPU
    tensor holding at least nbytes (of the stated dtype); the library sizes
    every access from the descriptor, so a short buffer would be overrun.
    Raw integer addresses are the caller's responsibility and pass as is."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and str(t.dtype) != "torch." + _DTYPE_NAMES[dtype]:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, the call needs {nbytes}")


def _check_conv_buffers(desc: conv3d_desc, x, w_packed, epi: Optional[conv3d_epilogue], y,
                        y_bytes: Optional[int] = None) -> None:
    esz = 1 if desc.dtype == FP8_E4M3 else 2
    od = conv3d_output_dims(desc)
    out_bytes = desc.n * od[0] * od[1] * od[2] * desc.cout * 2
    _check_buffer(x, desc.n * desc.d * desc.h * desc.w * desc.cin * esz, "x")
    pw = (conv3d_packed_weight_bytes_fp8 if esz == 1 else conv3d_packed_weight_bytes)(
        desc.cout, desc.cin)
    _check_buffer(w_packed, pw, "w_packed")
    _check_buffer(y, out_bytes if y_bytes is None else y_bytes, "y", "bf16")
    if epi is not None:
        t = getattr(epi, "tensors", {})
        _check_buffer(t.get("bias"), 4 * desc.cout, "bias", "fp32")
        _check_buffer(t.get("gamma"), 2 * desc.cout, "gamma", "bf16")
        _check_buffer(t.get("residual"), out_bytes, "residual", "bf16")
        _check_buffer(t.get("residual_out"), out_bytes, "residual_out", "bf16")


def _check_workspace(workspace, workspace_bytes: int) -> None:
    if workspace is not None and not isinstance(workspace, int):
        _check_buffer(workspace, workspace_bytes, "workspace")


# --------------------------------------------------------------------------- C entry points

def conv3d_packed_weight_bytes(cout: int, cin: int) -> int:
    return int(lib().conv3d_packed_weight_bytes(cout, cin))


def conv3d_pack_weight(w_oidhw, w_packed, cout: int, cin: int, stream=None) -> None:
    _check(lib().conv3d_pack_weight(_ptr(w_oidhw), _ptr(w_packed), cout, cin, _stream(stream)),
           "conv3d_pack_weight")


def conv3d_packed_weight_bytes_fp8(cout: int, cin: int) -> int:
    return int(lib().conv3d_packed_weight_bytes_fp8(cout, cin))


def conv3d_pack_weight_fp8(w_oidhw, w_packed, cout: int, cin: int, stream=None) -> None:
    _check(lib().conv3d_pack_weight_fp8(_ptr(w_oidhw), _ptr(w_packed), cout, cin, _stream(stream)),
           "conv3d_pack_weight_fp8")


def conv3d_pack_weight_2d(w_oihw, w_packed, cout: int, cin: int, stream=None) -> None:
    _check(lib().conv3d_pack_weight_2d(_ptr(w_oihw), _ptr(w_packed), cout, cin, _stream(stream)),
           "conv3d_pack_weight_2d")


def conv3d_output_dims(desc: conv3d_desc):
    out = (ctypes.c_int * 3)()
    _check(lib().conv3d_output_dims(ctypes.byref(desc), ctypes.byref(out)), "conv3d_output_dims")
    return tuple(out)


def conv3d_workspace_bytes(desc: conv3d_desc, epi: Optional[conv3d_epilogue] = None) -> int:
    out = ctypes.c_size_t()
    _check(lib().conv3d_workspace_bytes(ctypes.byref(desc), ctypes.byref(epi) if epi else None,
                                        ctypes.byref(out)), "conv3d_workspace_bytes")
    return int(out.value)


def conv3d_fwd(desc: conv3d_desc, x, w_packed, epi: Optional[conv3d_epilogue], y,
               workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    if workspace is not None and not workspace_bytes and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check_conv_buffers(desc, x, w_packed, epi, y)
    _check_workspace(workspace, workspace_bytes)
    _check(lib().conv3d_fwd(ctypes.byref(desc), _ptr(x), _ptr(w_packed),
                            ctypes.byref(epi) if epi else None, _ptr(y), _ptr(workspace),
                            workspace_bytes, _stream(stream)), "conv3d_fwd")


def conv3d_fwd_noalloc(desc: conv3d_desc, x, w_packed, epi: Optional[conv3d_epilogue], y,
                       stream=None) -> None:
    """conv3d_fwd without a workspace: the library's fixed per-device
    scratch serves instead (calls on one GPU must not overlap in time)."""
    _check_conv_buffers(desc, x, w_packed, epi, y)
    _check(lib().conv3d_fwd_noalloc(ctypes.byref(desc), _ptr(x), _ptr(w_packed),
                                    ctypes.byref(epi) if epi else None, _ptr(y),
                                    _stream(stream)), "conv3d_fwd_noalloc")


def conv3d_transpose(src, src_layout: int, dst, n: int, c: int, d: int, h: int, w: int,
                     stream=None) -> None:
    _check(lib().conv3d_transpose(_ptr(src), src_layout, _ptr(dst), n, c, d, h, w,
                                  _stream(stream)), "conv3d_transpose")


def conv3d_plan_describe(desc: conv3d_desc, epi: Optional[conv3d_epilogue] = None) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib().conv3d_plan_describe(ctypes.byref(desc), ctypes.byref(epi) if epi else None,
                                      buf, 512), "conv3d_plan_describe")
    return buf.value.decode()


def make_group_norm_desc(x_shape: Sequence[int], groups: int, *, eps: float = 1e-5,
                         silu: bool = False, t_isolated: bool = True) -> conv3d_group_norm_desc:
    """GroupNorm descriptor for an NDHWC tensor of shape x_shape."""
    n, d, h, w, c = x_shape
    return conv3d_group_norm_desc(n, d, h, w, c, groups, int(bool(t_isolated)), int(bool(silu)),
                                  eps)


def conv3d_group_norm_workspace_bytes(desc: conv3d_group_norm_desc) -> int:
    out = ctypes.c_size_t()
    _check(lib().conv3d_group_norm_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)),
           "conv3d_group_norm_workspace_bytes")
    return int(out.value)


def conv3d_group_norm(desc: conv3d_group_norm_desc, x, gamma, beta, y, workspace=None,
                      workspace_bytes: int = 0, stream=None) -> None:
    if workspace is not None and not workspace_bytes and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().conv3d_group_norm(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y),
                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "conv3d_group_norm")


def conv3d_gn_partials_bytes(desc: conv3d_desc) -> int:
    out = ctypes.c_size_t()
    _check(lib().conv3d_gn_partials_bytes(ctypes.byref(desc), ctypes.byref(out)),
           "conv3d_gn_partials_bytes")
    return int(out.value)


def conv3d_fwd_gn_stats(desc: conv3d_desc, x, w_packed, y, gn_partials, workspace=None,
                        workspace_bytes: int = 0, stream=None) -> None:
    """conv3d_fwd with no epilogue, plus the GroupNorm partial statistics of y."""
    if workspace is not None and not workspace_bytes and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check_conv_buffers(desc, x, w_packed, None, y)
    _check_workspace(workspace, workspace_bytes)
    _check_buffer(gn_partials, conv3d_gn_partials_bytes(desc), "gn_partials", "fp32")
    _check(lib().conv3d_fwd_gn_stats(ctypes.byref(desc), _ptr(x), _ptr(w_packed), _ptr(y),
                                     _ptr(gn_partials), _ptr(workspace), workspace_bytes,
                                     _stream(stream)), "conv3d_fwd_gn_stats")


def conv3d_group_norm_from_partials(desc: conv3d_group_norm_desc, conv: conv3d_desc,
                                    gn_partials, x, gamma, beta, y, workspace=None,
                                    workspace_bytes: int = 0, stream=None) -> None:
    """GroupNorm of a conv3d_fwd_gn_stats output from its partial statistics."""
    if workspace is not None and not workspace_bytes and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().conv3d_group_norm_from_partials(ctypes.byref(desc), ctypes.byref(conv),
                                                 _ptr(gn_partials), _ptr(x), _ptr(gamma),
                                                 _ptr(beta), _ptr(y), _ptr(workspace),
                                                 workspace_bytes, _stream(stream)),
           "conv3d_group_norm_from_partials")


def make_out_pad(pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), history_frames: int = 0, cache=None,
                 cache_frames: int = 0) -> conv3d_out_pad:
    """Padded-output placement for conv3d_fwd_padded."""
    op = conv3d_out_pad((ctypes.c_int * 3)(*pad_lo), (ctypes.c_int * 3)(*pad_hi),
                        history_frames, cache_frames, _ptr(cache))
    op.cache_tensor = cache
    return op


def conv3d_padded_workspace_bytes(desc: conv3d_desc, epi: Optional[conv3d_epilogue],
                                  out_pad: Optional[conv3d_out_pad]) -> int:
    out = ctypes.c_size_t()
    _check(lib().conv3d_padded_workspace_bytes(ctypes.byref(desc),
                                               ctypes.byref(epi) if epi else None,
                                               ctypes.byref(out_pad) if out_pad else None,
                                               ctypes.byref(out)), "conv3d_padded_workspace_bytes")
    return int(out.value)


def conv3d_fwd_padded(desc: conv3d_desc, x, w_packed, epi: Optional[conv3d_epilogue],
                      out_pad: Optional[conv3d_out_pad], y, workspace=None,
                      workspace_bytes: int = 0, stream=None) -> None:
    if workspace is not None and not workspace_bytes and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
    y_bytes = None
    if out_pad is not None:
        od = conv3d_output_dims(desc)
        y_bytes = desc.n * desc.cout * 2
        for i in range(3):
            y_bytes *= od[i] + out_pad.pad_lo[i] + out_pad.pad_hi[i]
        cache = getattr(out_pad, "cache_tensor", None)
        if out_pad.cache:
            _check_buffer(cache, desc.n * out_pad.cache_frames * od[1] * od[2] * desc.cout * 2,
                          "cache", "bf16")
    _check_conv_buffers(desc, x, w_packed, epi, y, y_bytes)
    _check_workspace(workspace, workspace_bytes)
    _check(lib().conv3d_fwd_padded(ctypes.byref(desc), _ptr(x), _ptr(w_packed),
                                   ctypes.byref(epi) if epi else None,
                                   ctypes.byref(out_pad) if out_pad else None, _ptr(y),
                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "conv3d_fwd_padded")


def conv3d_stream_pack_input(chunk, strides: Sequence[int], n: int, c: int, t: int, h: int, w: int,
                             history, history_frames: int, padded, c_pad: int, cache,
                             cache_frames: int, stream=None) -> None:
    st = (ctypes.c_longlong * 5)(*[int(v) for v in strides])
    _check(lib().conv3d_stream_pack_input(_ptr(chunk), ctypes.byref(st), n, c, t, h, w,
                                          _ptr(history), history_frames, _ptr(padded), c_pad,
                                          _ptr(cache), cache_frames, _stream(stream)),
           "conv3d_stream_pack_input")


def conv3d_norm_silu(x, n: int, d: int, h: int, w: int, c: int, epi: conv3d_epilogue,
                     out_pad: Optional[conv3d_out_pad], previous, y, stream=None) -> None:
    _check(lib().conv3d_norm_silu(_ptr(x), n, d, h, w, c, ctypes.byref(epi),
                                  ctypes.byref(out_pad) if out_pad else None, _ptr(previous), _ptr(y),
                                  _stream(stream)), "conv3d_norm_silu")
