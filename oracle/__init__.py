"""CPU oracle for the pool_stencil operations -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library.

The arithmetic lives in `oracle.c` (plain C, double precision, OpenMP over
the outer loops); this module only marshals numpy arrays into it.  Each
wrapper returns float64 arrays (float32 for the standalone max-pool, whose
result is exactly one of its float32 inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i, d, p, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64
    lib.or_window_out_dim.argtypes = [i, i, i, i, i]
    lib.or_window_out_dim.restype = i
    lib.or_convT_out_dim.argtypes = [i, i, i, i, i, i]
    lib.or_convT_out_dim.restype = i
    lib.or_num_threads.restype = i
    lib.or_conv2d.argtypes = [p, p, p, p] + [i] * 10
    lib.or_maxpool2d_f64.argtypes = [p, p] + [i] * 8
    lib.or_maxpool2d_f32.argtypes = [p, p] + [i] * 8
    lib.or_conv_tanh_scale_bias_maxpool.argtypes = [p, p, p, p, p] + [i] * 10 + [d] + [i] * 4
    lib.or_conv_tanh_scale_bias_maxpool_points.argtypes = (
        [p, p, p, p] + [i] * 10 + [d] + [i] * 4 + [i64, p, p])
    lib.or_tanh_scale_bias_maxpool.argtypes = [p, p, p] + [i] * 4 + [d] + [i] * 4
    lib.or_softmax_bias_scale_sigmoid.argtypes = [p, p, p] + [i] * 4 + [d]
    lib.or_conv_transpose2d.argtypes = [p, p, p, p] + [i] * 10
    lib.or_convT_softmax_bias_scale_sigmoid.argtypes = [p, p, p, p, p] + [i] * 10 + [d]
    lib.or_convT_softmax_bias_scale_sigmoid_pixels.argtypes = (
        [p, p, p, p] + [i] * 10 + [d] + [i64, p, p])
    _lib = lib
    return lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return _load().or_num_threads()


def window_out_dim(n, k, s, p, d=1) -> int:
    return _load().or_window_out_dim(n, k, s, p, d)


def convT_out_dim(n, k, s, p, op, d=1) -> int:
    return _load().or_convT_out_dim(n, k, s, p, op, d)


def conv2d(x, w, bias=None, stride=1, pad=0, dil=1):
    x, w = _f32(x), _f32(w)
    b = None if bias is None else _f32(bias)
    N, Cin, H, W = x.shape
    Cout, _, kH, kW = w.shape
    OH, OW = window_out_dim(H, kH, stride, pad, dil), window_out_dim(W, kW, stride, pad, dil)
    y = np.zeros((N, Cout, max(OH, 0), max(OW, 0)), dtype=np.float64)
    _load().or_conv2d(_ptr(x), _ptr(w), _ptr(b), _ptr(y), N, Cin, H, W, Cout, kH, kW,
                      stride, pad, dil)
    return y


def maxpool2d(x, k, stride=None, pad=0, dil=1):
    """Max-pool of float32 (returns float32) or float64 (returns float64) data."""
    stride = k if stride is None or stride <= 0 else stride
    N, C, H, W = x.shape
    OH, OW = window_out_dim(H, k, stride, pad, dil), window_out_dim(W, k, stride, pad, dil)
    if x.dtype == np.float64:
        x = np.ascontiguousarray(x)
        y = np.zeros((N, C, max(OH, 0), max(OW, 0)), dtype=np.float64)
        _load().or_maxpool2d_f64(_ptr(x), _ptr(y), N, C, H, W, k, stride, pad, dil)
    else:
        x = _f32(x)
        y = np.zeros((N, C, max(OH, 0), max(OW, 0)), dtype=np.float32)
        _load().or_maxpool2d_f32(_ptr(x), _ptr(y), N, C, H, W, k, stride, pad, dil)
    return y


def _conv_pool_args(c):
    x, w = _f32(c["x"]), _f32(c["w"])
    cb = None if c.get("conv_bias") is None else _f32(c["conv_bias"])
    b2 = _f32(c["bias2"])
    ps = c["pool_stride"] if c["pool_stride"] > 0 else c["pool_k"]
    return x, w, cb, b2, ps


def conv_pool_out_shape(c):
    ps = c["pool_stride"] if c["pool_stride"] > 0 else c["pool_k"]
    OH = window_out_dim(c["H"], c["kH"], c["conv_stride"], c["conv_pad"], c["conv_dil"])
    OW = window_out_dim(c["W"], c["kW"], c["conv_stride"], c["conv_pad"], c["conv_dil"])
    PH = window_out_dim(OH, c["pool_k"], ps, c["pool_pad"], c["pool_dil"])
    PW = window_out_dim(OW, c["pool_k"], ps, c["pool_pad"], c["pool_dil"])
    return (c["N"], c["Cout"], PH, PW)


def conv_tanh_scale_bias_maxpool(c):
    """Full fused op for a case dict (see inputgen); float64 [N,Cout,PH,PW]."""
    x, w, cb, b2, ps = _conv_pool_args(c)
    out = np.zeros(conv_pool_out_shape(c), dtype=np.float64)
    _load().or_conv_tanh_scale_bias_maxpool(
        _ptr(x), _ptr(w), _ptr(cb), _ptr(b2), _ptr(out),
        c["N"], c["Cin"], c["H"], c["W"], c["Cout"], c["kH"], c["kW"],
        c["conv_stride"], c["conv_pad"], c["conv_dil"], float(c["scale"]),
        c["pool_k"], ps, c["pool_pad"], c["pool_dil"])
    return out


def conv_tanh_scale_bias_maxpool_points(c, flat_idx):
    """Fused op at selected flat output indices; float64 [len(flat_idx)]."""
    x, w, cb, b2, ps = _conv_pool_args(c)
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64)
    out = np.zeros(idx.shape[0], dtype=np.float64)
    _load().or_conv_tanh_scale_bias_maxpool_points(
        _ptr(x), _ptr(w), _ptr(cb), _ptr(b2),
        c["N"], c["Cin"], c["H"], c["W"], c["Cout"], c["kH"], c["kW"],
        c["conv_stride"], c["conv_pad"], c["conv_dil"], float(c["scale"]),
        c["pool_k"], ps, c["pool_pad"], c["pool_dil"], idx.shape[0], _ptr(idx), _ptr(out))
    return out


def tanh_scale_bias_maxpool(y, bias2, scale, k, stride=None, pad=0, dil=1):
    """maxpool(tanh(y) * scale + bias2[c]) of a stored float32 conv output; float64."""
    y, b2 = _f32(y), _f32(bias2)
    stride = k if stride is None or stride <= 0 else stride
    N, C, H, W = y.shape
    OH, OW = window_out_dim(H, k, stride, pad, dil), window_out_dim(W, k, stride, pad, dil)
    out = np.zeros((N, C, max(OH, 0), max(OW, 0)), dtype=np.float64)
    _load().or_tanh_scale_bias_maxpool(_ptr(y), _ptr(b2), _ptr(out), N, C, H, W, float(scale),
                                       k, stride, pad, dil)
    return out


def softmax_bias_scale_sigmoid(y, bias2, scale):
    """sigmoid((softmax_c(y) + bias2[c]) * scale) of a stored float32 convT output; float64."""
    y, b2 = _f32(y), _f32(bias2)
    N, C, H, W = y.shape
    out = np.zeros(y.shape, dtype=np.float64)
    _load().or_softmax_bias_scale_sigmoid(_ptr(y), _ptr(b2), _ptr(out), N, C, H, W,
                                          float(scale))
    return out


def conv_transpose2d(x, w, bias=None, stride=2, pad=1, output_padding=0, dil=1):
    x, w = _f32(x), _f32(w)
    b = None if bias is None else _f32(bias)
    N, Cin, H, W = x.shape
    _, Cout, k, _ = w.shape
    OH = convT_out_dim(H, k, stride, pad, output_padding, dil)
    OW = convT_out_dim(W, k, stride, pad, output_padding, dil)
    y = np.zeros((N, Cout, max(OH, 0), max(OW, 0)), dtype=np.float64)
    _load().or_conv_transpose2d(_ptr(x), _ptr(w), _ptr(b), _ptr(y), N, Cin, H, W, Cout, k,
                                stride, pad, output_padding, dil)
    return y


def convT_out_shape(c):
    OH = convT_out_dim(c["H"], c["k"], c["stride"], c["pad"], c["output_padding"], c["dil"])
    OW = convT_out_dim(c["W"], c["k"], c["stride"], c["pad"], c["output_padding"], c["dil"])
    return (c["N"], c["Cout"], OH, OW)


def _convT_args(c):
    x, w = _f32(c["x"]), _f32(c["w"])
    cb = None if c.get("convT_bias") is None else _f32(c["convT_bias"])
    return x, w, cb, _f32(c["bias2"])


def convT_softmax_bias_scale_sigmoid(c):
    x, w, cb, b2 = _convT_args(c)
    out = np.zeros(convT_out_shape(c), dtype=np.float64)
    _load().or_convT_softmax_bias_scale_sigmoid(
        _ptr(x), _ptr(w), _ptr(cb), _ptr(b2), _ptr(out),
        c["N"], c["Cin"], c["H"], c["W"], c["Cout"], c["k"], c["stride"], c["pad"],
        c["output_padding"], c["dil"], float(c["scale"]))
    return out


def convT_softmax_bias_scale_sigmoid_pixels(c, flat_pix):
    """All Cout outputs at selected pixels (flat n*OH*OW + oh*OW + ow); float64 [npix, Cout]."""
    x, w, cb, b2 = _convT_args(c)
    pix = np.ascontiguousarray(flat_pix, dtype=np.int64)
    out = np.zeros((pix.shape[0], c["Cout"]), dtype=np.float64)
    _load().or_convT_softmax_bias_scale_sigmoid_pixels(
        _ptr(x), _ptr(w), _ptr(cb), _ptr(b2),
        c["N"], c["Cin"], c["H"], c["W"], c["Cout"], c["k"], c["stride"], c["pad"],
        c["output_padding"], c["dil"], float(c["scale"]), pix.shape[0], _ptr(pix), _ptr(out))
    return out
