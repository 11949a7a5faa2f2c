"""Python binding of libpool_stencil (fused sliding-window stencils for MI355X).

Thin ctypes layer over the C ABI declared in include/pool_stencil.h: it checks
tensor placement/dtype/contiguity, allocates outputs with torch (device memory
only), passes raw device pointers and torch's current HIP stream, and turns a
non-zero status into PsError.  Every step of every operation runs in the HIP
kernels of the library; there is no other implementation to fall back to, and
importing this package fails if the library has not been built.

Operations (same names as the C entry points, without the ps_ prefix):
    conv_tanh_scale_bias_maxpool(x, w, conv_bias, bias2, scale, pool_k, ...)
    conv2d(x, w, bias=None, stride=1, pad=0, dil=1)
    maxpool2d(x, k, stride=None, pad=0, dil=1)
    convT_softmax_bias_scale_sigmoid(x, w, convT_bias, bias2, scale, ...)
    convT2d(x, w, bias=None, stride=2, pad=1, output_padding=1, dil=1)
    tanh_scale_bias_maxpool(y, bias2, scale, k, stride=None, pad=0, dil=1)
    softmax_bias_scale_sigmoid(y, bias2, scale, out=None)   (out=y: in place)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpool_stencil.so")

PS_OK, PS_ERR_NULL, PS_ERR_SHAPE, PS_ERR_PARAM, PS_ERR_UNSUPPORTED, PS_ERR_ALIGN, PS_ERR_HIP = range(7)
PS_F32, PS_BF16 = 0, 1

# Every symbol include/pool_stencil.h declares.
EXPORTS = (
    "ps_status_string", "ps_version", "ps_conv2d_out_dim", "ps_pool2d_out_dim",
    "ps_convT2d_out_dim", "ps_conv_tanh_scale_bias_maxpool", "ps_conv2d", "ps_maxpool2d",
    "ps_convT_softmax_bias_scale_sigmoid", "ps_convT_softmax_bias_scale_sigmoid_bf16",
    "ps_convT2d", "ps_tanh_scale_bias_maxpool", "ps_softmax_bias_scale_sigmoid",
)


class PsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (libamdhip64).  Importing torch first makes the
    # dynamic loader resolve the library's libamdhip64.so.7 dependency to that same
    # runtime; loading the library first would map a second, independent runtime that
    # cannot see torch's allocations or streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python pool_stencil_amd/build.py` "
            "(or __graft_entry__.build()) before using pool_stencil_amd")
    lib = ctypes.CDLL(LIB_PATH)
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.ps_status_string.argtypes = [i]
    lib.ps_status_string.restype = ctypes.c_char_p
    lib.ps_version.restype = i
    lib.ps_conv2d_out_dim.argtypes = [i, i, i, i, i, ctypes.POINTER(i)]
    lib.ps_pool2d_out_dim.argtypes = [i, i, i, i, i, ctypes.POINTER(i)]
    lib.ps_convT2d_out_dim.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i)]
    lib.ps_conv_tanh_scale_bias_maxpool.argtypes = [p, p, p, p, p] + [i] * 11 + [f] + [i] * 4 + [p]
    lib.ps_conv2d.argtypes = [p, p, p, p] + [i] * 11 + [p]
    lib.ps_maxpool2d.argtypes = [p, p] + [i] * 8 + [p]
    lib.ps_convT_softmax_bias_scale_sigmoid.argtypes = [p, p, p, p, p] + [i] * 10 + [f, p]
    lib.ps_convT_softmax_bias_scale_sigmoid_bf16.argtypes = [p, p, p, p, p] + [i] * 10 + [f, p]
    lib.ps_convT2d.argtypes = [p, p, p, p] + [i] * 10 + [p]
    lib.ps_tanh_scale_bias_maxpool.argtypes = [p, p, p] + [i] * 5 + [f] + [i] * 4 + [p]
    lib.ps_softmax_bias_scale_sigmoid.argtypes = [p, p, p] + [i] * 4 + [f, p]
    for name in ("ps_conv2d_out_dim", "ps_pool2d_out_dim", "ps_convT2d_out_dim",
                 "ps_conv_tanh_scale_bias_maxpool", "ps_conv2d", "ps_maxpool2d",
                 "ps_convT_softmax_bias_scale_sigmoid",
                 "ps_convT_softmax_bias_scale_sigmoid_bf16", "ps_convT2d",
                 "ps_tanh_scale_bias_maxpool", "ps_softmax_bias_scale_sigmoid"):
        getattr(lib, name).restype = i
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    """The loaded C library (for tests that call the ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.ps_status_string(int(status)).decode()


def version() -> int:
    return _lib.ps_version()


def _dim(fn, *args) -> int:
    out = ctypes.c_int(-1)
    st = fn(*[int(a) for a in args], ctypes.byref(out))
    if st != PS_OK:
        raise PsError(st, fn.__name__)
    return out.value


def conv2d_out_dim(n, k, stride=1, pad=0, dil=1) -> int:
    return _dim(_lib.ps_conv2d_out_dim, n, k, stride, pad, dil)


def pool2d_out_dim(n, k, stride=None, pad=0, dil=1) -> int:
    return _dim(_lib.ps_pool2d_out_dim, n, k, 0 if stride is None else stride, pad, dil)


def convT2d_out_dim(n, k, stride, pad, output_padding, dil=1) -> int:
    return _dim(_lib.ps_convT2d_out_dim, n, k, stride, pad, output_padding, dil)


# ------------------------------------------------------------------ tensors --
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t, name, dtypes, device=None):
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (NCHW)")


def conv_tanh_scale_bias_maxpool(x, w, conv_bias, bias2, scale, pool_k, pool_stride=None,
                                 conv_stride=1, conv_pad=0, conv_dil=1, pool_pad=0, pool_dil=1,
                                 out=None, stream=None):
    """maxpool(tanh(conv2d(x, w, conv_bias)) * scale + bias2[c]) in one fused kernel.

    x [N,Cin,H,W] and w [Cout,Cin,kH,kW] share a dtype (float32 or bfloat16);
    conv_bias (optional) and bias2 [Cout] (any shape with Cout elements, e.g. [Cout,1,1])
    are float32.  Returns [N,Cout,PH,PW] in x's dtype."""
    torch = _torch()
    _check(x, "x", (torch.float32, torch.bfloat16))
    _check(w, "w", (x.dtype,), x.device)
    _check(conv_bias, "conv_bias", (torch.float32,), x.device)
    _check(bias2, "bias2", (torch.float32,), x.device)
    N, Cin, H, W = x.shape
    Cout, Cin_w, kH, kW = w.shape
    if Cin_w != Cin:
        raise ValueError(f"w has {Cin_w} input channels, x has {Cin}")
    if bias2.numel() != Cout or (conv_bias is not None and conv_bias.numel() != Cout):
        raise ValueError("bias vectors must hold Cout elements")
    ps = 0 if pool_stride is None else pool_stride
    OH = conv2d_out_dim(H, kH, conv_stride, conv_pad, conv_dil)
    OW = conv2d_out_dim(W, kW, conv_stride, conv_pad, conv_dil)
    PH = pool2d_out_dim(OH, pool_k, pool_stride, pool_pad, pool_dil)
    PW = pool2d_out_dim(OW, pool_k, pool_stride, pool_pad, pool_dil)
    if out is None:
        out = torch.empty((N, Cout, PH, PW), dtype=x.dtype, device=x.device)
    else:
        _check(out, "out", (x.dtype,), x.device)
        if tuple(out.shape) != (N, Cout, PH, PW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, Cout, PH, PW)}")
    dtype = PS_BF16 if x.dtype == torch.bfloat16 else PS_F32
    st = _lib.ps_conv_tanh_scale_bias_maxpool(
        _ptr(x), _ptr(w), _ptr(conv_bias), _ptr(bias2), _ptr(out), dtype, N, Cin, H, W, Cout,
        kH, kW, conv_stride, conv_pad, conv_dil, float(scale), pool_k, ps, pool_pad, pool_dil,
        _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_conv_tanh_scale_bias_maxpool")
    return out


def conv2d(x, w, bias=None, stride=1, pad=0, dil=1, out=None, stream=None):
    """Conv2d + bias (cross-correlation, zero padding) of an NCHW tensor.

    x [N,Cin,H,W] and w [Cout,Cin,kH,kW] share a dtype (float32 or bfloat16); bias
    (optional) is float32 [Cout].  Returns [N,Cout,OH,OW] in x's dtype."""
    torch = _torch()
    _check(x, "x", (torch.float32, torch.bfloat16))
    _check(w, "w", (x.dtype,), x.device)
    _check(bias, "bias", (torch.float32,), x.device)
    N, Cin, H, W = x.shape
    Cout, Cin_w, kH, kW = w.shape
    if Cin_w != Cin:
        raise ValueError(f"w has {Cin_w} input channels, x has {Cin}")
    if bias is not None and bias.numel() != Cout:
        raise ValueError("bias must hold Cout elements")
    OH = conv2d_out_dim(H, kH, stride, pad, dil)
    OW = conv2d_out_dim(W, kW, stride, pad, dil)
    if out is None:
        out = torch.empty((N, Cout, OH, OW), dtype=x.dtype, device=x.device)
    else:
        _check(out, "out", (x.dtype,), x.device)
        if tuple(out.shape) != (N, Cout, OH, OW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, Cout, OH, OW)}")
    dtype = PS_BF16 if x.dtype == torch.bfloat16 else PS_F32
    st = _lib.ps_conv2d(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), dtype, N, Cin, H, W, Cout,
                        kH, kW, stride, pad, dil, _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_conv2d")
    return out


def maxpool2d(x, k, stride=None, pad=0, dil=1, out=None, stream=None):
    """MaxPool2d (floor mode, -inf padding) of a float32 NCHW tensor."""
    torch = _torch()
    _check(x, "x", (torch.float32,))
    N, C, H, W = x.shape
    OH = pool2d_out_dim(H, k, stride, pad, dil)
    OW = pool2d_out_dim(W, k, stride, pad, dil)
    if out is None:
        out = torch.empty((N, C, OH, OW), dtype=torch.float32, device=x.device)
    else:
        _check(out, "out", (torch.float32,), x.device)
        if tuple(out.shape) != (N, C, OH, OW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, C, OH, OW)}")
    st = _lib.ps_maxpool2d(_ptr(x), _ptr(out), N, C, H, W, k, 0 if stride is None else stride,
                           pad, dil, _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_maxpool2d")
    return out


def convT_softmax_bias_scale_sigmoid(x, w, convT_bias, bias2, scale, stride=2, pad=1,
                                     output_padding=1, dil=1, out=None, stream=None):
    """sigmoid((softmax_c(conv_transpose2d(x, w, convT_bias)) + bias2[c]) * scale), fused.

    x [N,Cin,H,W] and w [Cin,Cout,k,k] (PyTorch's ConvTranspose2d layout) share a
    dtype, float32 or bfloat16 (bf16: fp32 accumulation, output in bf16); the biases
    are float32."""
    torch = _torch()
    _check(x, "x", (torch.float32, torch.bfloat16))
    _check(w, "w", (x.dtype,), x.device)
    _check(convT_bias, "convT_bias", (torch.float32,), x.device)
    _check(bias2, "bias2", (torch.float32,), x.device)
    N, Cin, H, W = x.shape
    Cin_w, Cout, k, k2 = w.shape
    if Cin_w != Cin or k != k2:
        raise ValueError("w must be [Cin, Cout, k, k]")
    if bias2.numel() != Cout or (convT_bias is not None and convT_bias.numel() != Cout):
        raise ValueError("bias vectors must hold Cout elements")
    OH = convT2d_out_dim(H, k, stride, pad, output_padding, dil)
    OW = convT2d_out_dim(W, k, stride, pad, output_padding, dil)
    if out is None:
        out = torch.empty((N, Cout, OH, OW), dtype=x.dtype, device=x.device)
    else:
        _check(out, "out", (x.dtype,), x.device)
        if tuple(out.shape) != (N, Cout, OH, OW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, Cout, OH, OW)}")
    fn = (_lib.ps_convT_softmax_bias_scale_sigmoid_bf16 if x.dtype == torch.bfloat16
          else _lib.ps_convT_softmax_bias_scale_sigmoid)
    st = fn(_ptr(x), _ptr(w), _ptr(convT_bias), _ptr(bias2), _ptr(out), N, Cin, H, W, Cout, k,
            stride, pad, output_padding, dil, float(scale), _stream(stream))
    if st != PS_OK:
        raise PsError(st, fn.__name__)
    return out


def convT2d(x, w, bias=None, stride=2, pad=1, output_padding=1, dil=1, out=None, stream=None):
    """ConvTranspose2d + bias: x [N,Cin,H,W] float32, w [Cin,Cout,k,k] float32."""
    torch = _torch()
    _check(x, "x", (torch.float32,))
    _check(w, "w", (torch.float32,), x.device)
    _check(bias, "bias", (torch.float32,), x.device)
    N, Cin, H, W = x.shape
    Cin_w, Cout, k, k2 = w.shape
    if Cin_w != Cin or k != k2:
        raise ValueError("w must be [Cin, Cout, k, k]")
    if bias is not None and bias.numel() != Cout:
        raise ValueError("bias must hold Cout elements")
    OH = convT2d_out_dim(H, k, stride, pad, output_padding, dil)
    OW = convT2d_out_dim(W, k, stride, pad, output_padding, dil)
    if out is None:
        out = torch.empty((N, Cout, OH, OW), dtype=torch.float32, device=x.device)
    else:
        _check(out, "out", (torch.float32,), x.device)
        if tuple(out.shape) != (N, Cout, OH, OW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, Cout, OH, OW)}")
    st = _lib.ps_convT2d(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), N, Cin, H, W, Cout, k, stride,
                         pad, output_padding, dil, _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_convT2d")
    return out


def tanh_scale_bias_maxpool(y, bias2, scale, k, stride=None, pad=0, dil=1, out=None,
                            stream=None):
    """maxpool(tanh(y) * scale + bias2[c]) of a stored conv output y [N,C,H,W]
    (float32 or bfloat16; output in y's dtype)."""
    torch = _torch()
    _check(y, "y", (torch.float32, torch.bfloat16))
    _check(bias2, "bias2", (torch.float32,), y.device)
    N, C, H, W = y.shape
    if bias2.numel() != C:
        raise ValueError("bias2 must hold C elements")
    OH = pool2d_out_dim(H, k, stride, pad, dil)
    OW = pool2d_out_dim(W, k, stride, pad, dil)
    if out is None:
        out = torch.empty((N, C, OH, OW), dtype=y.dtype, device=y.device)
    else:
        _check(out, "out", (y.dtype,), y.device)
        if tuple(out.shape) != (N, C, OH, OW):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, C, OH, OW)}")
    dtype = PS_BF16 if y.dtype == torch.bfloat16 else PS_F32
    st = _lib.ps_tanh_scale_bias_maxpool(_ptr(y), _ptr(bias2), _ptr(out), dtype, N, C, H, W,
                                         float(scale), k, 0 if stride is None else stride, pad,
                                         dil, _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_tanh_scale_bias_maxpool")
    return out


def softmax_bias_scale_sigmoid(y, bias2, scale, out=None, stream=None):
    """sigmoid((softmax over channels of y + bias2[c]) * scale) of a stored float32
    y [N,C,H,W]; pass out=y to run in place."""
    torch = _torch()
    _check(y, "y", (torch.float32,))
    _check(bias2, "bias2", (torch.float32,), y.device)
    N, C, H, W = y.shape
    if bias2.numel() != C:
        raise ValueError("bias2 must hold C elements")
    if out is None:
        out = torch.empty_like(y)
    else:
        _check(out, "out", (torch.float32,), y.device)
        if out.shape != y.shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(y.shape)}")
    st = _lib.ps_softmax_bias_scale_sigmoid(_ptr(y), _ptr(bias2), _ptr(out), N, C, H, W,
                                            float(scale), _stream(stream))
    if st != PS_OK:
        raise PsError(st, "ps_softmax_bias_scale_sigmoid")
    return out
