"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments before touching a device.  No test
here launches a kernel (fake device pointers are only passed where validation
must reject the call first).  The tests that pass fake pointers run only where
no GPU is visible, so that a validation regression can never send them to a
kernel."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    # counting devices does not initialise the GPU runtime
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001 - no torch: no device either
        return False


fake_pointers = pytest.mark.skipif(
    _gpu_visible(), reason="passes fake device pointers; runs only where no GPU is visible")


@pytest.fixture(scope="module")
def ps():
    lib_path = os.path.join(ROOT, "pool_stencil_amd", "libpool_stencil.so")
    if not os.path.exists(lib_path):
        import __graft_entry__
        __graft_entry__.build()
    import pool_stencil_amd
    return pool_stencil_amd


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "pool_stencil.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ps_[A-Za-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported(ps):
    syms = _header_symbols()
    assert len(syms) >= 8
    assert set(syms) == set(ps.EXPORTS)
    lib = ps.lib()
    for s in syms:
        assert hasattr(lib, s), s


def test_no_undefined_kernel_handles(ps):
    """Every kernel the library launches is defined in it: the host pass of the compiler
    can drop a kernel's launch handle without a diagnostic, which would otherwise show
    only when the library is loaded on a device."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "ps_build", os.path.join(ROOT, "pool_stencil_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    assert build._undefined_own_symbols(ps.LIB_PATH) == []


def test_status_strings(ps):
    for st in range(7):
        s = ps.status_string(st)
        assert isinstance(s, str) and s
    assert ps.status_string(99) == "unknown status"
    assert ps.version() >= 100


@pytest.mark.parametrize("n,k,s,p,d", [(256, 3, 1, 0, 1), (254, 4, 4, 0, 1), (512, 4, 1, 1, 1),
                                       (129, 4, 2, 1, 1), (32, 3, 1, 0, 1), (30, 4, 4, 0, 1),
                                       (17, 5, 2, 2, 2), (7, 3, 3, 1, 1)])
def test_window_extent_matches_oracle(ps, n, k, s, p, d):
    assert ps.conv2d_out_dim(n, k, s, p, d) == oracle.window_out_dim(n, k, s, p, d)
    assert ps.pool2d_out_dim(n, k, s, p, d) == oracle.window_out_dim(n, k, s, p, d)


def test_pool_default_stride(ps):
    assert ps.pool2d_out_dim(254, 4) == 63


@pytest.mark.parametrize("n,k,s,p,op,d", [(64, 4, 2, 1, 1, 1), (64, 4, 2, 1, 0, 1),
                                          (5, 3, 3, 0, 2, 1), (4, 3, 2, 2, 1, 2)])
def test_transposed_extent_matches_oracle(ps, n, k, s, p, op, d):
    assert ps.convT2d_out_dim(n, k, s, p, op, d) == oracle.convT_out_dim(n, k, s, p, op, d)


def test_shape_query_errors(ps):
    lib = ps.lib()
    out = ctypes.c_int(-7)
    assert lib.ps_conv2d_out_dim(10, 3, 1, 0, 1, None) == ps.PS_ERR_NULL
    assert lib.ps_conv2d_out_dim(10, 0, 1, 0, 1, ctypes.byref(out)) == ps.PS_ERR_PARAM
    assert lib.ps_conv2d_out_dim(10, 3, 0, 0, 1, ctypes.byref(out)) == ps.PS_ERR_PARAM
    assert lib.ps_conv2d_out_dim(10, 3, 1, -1, 1, ctypes.byref(out)) == ps.PS_ERR_PARAM
    assert lib.ps_conv2d_out_dim(2, 3, 1, 0, 1, ctypes.byref(out)) == ps.PS_ERR_SHAPE
    assert lib.ps_conv2d_out_dim(0, 1, 1, 0, 1, ctypes.byref(out)) == ps.PS_ERR_SHAPE
    # extents past INT_MAX are rejected, not truncated (conv, and pool through it)
    int_max = 2**31 - 1
    assert lib.ps_conv2d_out_dim(int_max, 1, 1, 1, 1, ctypes.byref(out)) == ps.PS_ERR_SHAPE
    assert lib.ps_pool2d_out_dim(int_max, 1, 1, 1, 1, ctypes.byref(out)) == ps.PS_ERR_SHAPE
    assert lib.ps_convT2d_out_dim(int_max, 4, 2, 0, 0, 1, ctypes.byref(out)) == ps.PS_ERR_SHAPE
    assert out.value == -7  # untouched on error
    assert lib.ps_conv2d_out_dim(int_max, 3, 1, 1, 1, ctypes.byref(out)) == ps.PS_OK
    assert out.value == int_max
    # output_padding must be < max(stride, dilation)
    assert lib.ps_convT2d_out_dim(64, 4, 2, 1, 2, 1, ctypes.byref(out)) == ps.PS_ERR_PARAM
    assert lib.ps_convT2d_out_dim(64, 4, 2, 1, 1, 1, ctypes.byref(out)) == ps.PS_OK
    assert out.value == 129


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation rejects first
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def _conv(lib, x=FAKE, w=FAKE, cb=None, b2=FAKE, y=FAKE, dtype=0, N=2, Cin=8, H=32, W=32,
          Cout=16, kH=3, kW=3, cs=1, cp=0, cd=1, scale=2.0, pk=4, pst=0, pp=0, pd=1):
    return lib.ps_conv_tanh_scale_bias_maxpool(x, w, cb, b2, y, dtype, N, Cin, H, W, Cout, kH, kW,
                                               cs, cp, cd, scale, pk, pst, pp, pd, None)


@fake_pointers
def test_conv_pool_validation(ps):
    lib = ps.lib()
    assert _conv(lib, x=None) == ps.PS_ERR_NULL
    assert _conv(lib, b2=None) == ps.PS_ERR_NULL
    assert _conv(lib, dtype=7) == ps.PS_ERR_PARAM
    assert _conv(lib, N=0) == ps.PS_ERR_SHAPE
    assert _conv(lib, H=2) == ps.PS_ERR_SHAPE            # conv window does not fit
    assert _conv(lib, H=5) == ps.PS_ERR_SHAPE            # conv 3 rows < pool 4
    assert _conv(lib, cp=-1) == ps.PS_ERR_PARAM
    # Every other argument combination is covered by one of the two kernels; only a
    # pool window wider than 16 conv outputs and a conv kernel whose weights do not
    # fit the LDS of a compute unit remain unsupported.  (Supported combinations are
    # not exercised here: with the fake pointers they would launch a kernel.)
    assert _conv(lib, pk=17, H=40, W=40) == ps.PS_ERR_UNSUPPORTED
    assert _conv(lib, pk=9, pd=2, H=40, W=40) == ps.PS_ERR_UNSUPPORTED
    assert _conv(lib, kH=13, kW=13, pk=2, H=64, W=64) == ps.PS_ERR_UNSUPPORTED
    # one image of 2^31 bytes or more: the kernels' 32-bit byte offsets do not reach
    assert _conv(lib, H=8192, W=8192) == ps.PS_ERR_UNSUPPORTED                # fp32, 8 ch
    assert _conv(lib, dtype=1, Cin=16, H=8192, W=8192) == ps.PS_ERR_UNSUPPORTED  # bf16
    assert _conv(lib, x=MISALIGNED) == ps.PS_ERR_ALIGN
    assert _conv(lib, y=MISALIGNED) == ps.PS_ERR_ALIGN
    assert _conv(lib, kH=5, kW=5, y=MISALIGNED) == ps.PS_ERR_ALIGN


def _conv2d(lib, x=FAKE, w=FAKE, b=None, y=FAKE, dtype=0, N=1, Cin=8, H=16, W=16, Cout=16,
            kH=3, kW=3, s=1, p=0, d=1):
    return lib.ps_conv2d(x, w, b, y, dtype, N, Cin, H, W, Cout, kH, kW, s, p, d, None)


@fake_pointers
def test_conv2d_validation(ps):
    lib = ps.lib()
    assert _conv2d(lib, x=None) == ps.PS_ERR_NULL
    assert _conv2d(lib, y=None) == ps.PS_ERR_NULL
    assert _conv2d(lib, dtype=2) == ps.PS_ERR_PARAM
    assert _conv2d(lib, Cout=0) == ps.PS_ERR_SHAPE
    assert _conv2d(lib, H=2) == ps.PS_ERR_SHAPE
    assert _conv2d(lib, s=0) == ps.PS_ERR_PARAM
    assert _conv2d(lib, p=-1) == ps.PS_ERR_PARAM
    assert _conv2d(lib, d=0) == ps.PS_ERR_PARAM
    assert _conv2d(lib, w=MISALIGNED) == ps.PS_ERR_ALIGN
    assert _conv2d(lib, kH=13, kW=13, H=32, W=32) == ps.PS_ERR_UNSUPPORTED
    assert _conv2d(lib, N=1 << 20, Cin=1 << 20) == ps.PS_ERR_SHAPE


def _pool(lib, x=FAKE, y=FAKE, N=1, C=1, H=8, W=8, k=4, s=1, p=1, d=1):
    return lib.ps_maxpool2d(x, y, N, C, H, W, k, s, p, d, None)


@fake_pointers
def test_maxpool_validation(ps):
    lib = ps.lib()
    assert _pool(lib, x=None) == ps.PS_ERR_NULL
    assert _pool(lib, H=0) == ps.PS_ERR_SHAPE
    assert _pool(lib, k=0) == ps.PS_ERR_PARAM
    assert _pool(lib, p=-1) == ps.PS_ERR_PARAM
    assert _pool(lib, H=2, p=0) == ps.PS_ERR_SHAPE
    # a padding that takes window indices past 32 bits (a large stride keeps OH small)
    assert _pool(lib, H=8, W=8, k=3, s=1 << 20, p=1 << 30) == ps.PS_ERR_UNSUPPORTED
    assert _pool(lib, y=MISALIGNED) == ps.PS_ERR_ALIGN
    assert _pool(lib, N=1 << 20, C=1 << 20) == ps.PS_ERR_SHAPE   # > 2^40 elements


def _convT(lib, x=FAKE, w=FAKE, cb=None, b2=FAKE, y=FAKE, N=1, Cin=64, H=8, W=8, Cout=128, k=4,
           s=2, p=1, op=1, d=1, scale=2.0):
    return lib.ps_convT_softmax_bias_scale_sigmoid(x, w, cb, b2, y, N, Cin, H, W, Cout, k, s, p,
                                                   op, d, scale, None)


@fake_pointers
def test_convT_validation(ps):
    lib = ps.lib()
    assert _convT(lib, w=None) == ps.PS_ERR_NULL
    assert _convT(lib, Cout=0) == ps.PS_ERR_SHAPE
    assert _convT(lib, op=2) == ps.PS_ERR_PARAM
    assert _convT(lib, k=3) == ps.PS_ERR_UNSUPPORTED
    assert _convT(lib, s=3) == ps.PS_ERR_UNSUPPORTED
    assert _convT(lib, Cout=272) == ps.PS_ERR_UNSUPPORTED
    assert _convT(lib, Cin=80) == ps.PS_ERR_UNSUPPORTED     # a class's weights exceed the LDS
    assert _convT(lib, Cout=160) == ps.PS_ERR_UNSUPPORTED   # likewise at Cin = 64
    assert _convT(lib, Cout=256, Cin=40) == ps.PS_ERR_UNSUPPORTED
    assert _convT(lib, p=5, H=2, W=2, op=0) == ps.PS_ERR_SHAPE   # (2-1)*2 - 10 + 4 < 1
    assert _convT(lib, Cin=76, Cout=128, N=1 << 12, H=64, W=64) == ps.PS_ERR_UNSUPPORTED  # >= 2^29
    assert _convT(lib, x=MISALIGNED) == ps.PS_ERR_ALIGN


@fake_pointers
def test_convT2d_validation(ps):
    lib = ps.lib()

    def call(x=FAKE, w=FAKE, b=None, y=FAKE, N=1, Cin=64, H=8, W=8, Cout=128, k=4, s=2, p=1,
             op=1, d=1):
        return lib.ps_convT2d(x, w, b, y, N, Cin, H, W, Cout, k, s, p, op, d, None)

    assert call(y=None) == ps.PS_ERR_NULL
    assert call(H=0) == ps.PS_ERR_SHAPE
    assert call(op=2) == ps.PS_ERR_PARAM
    assert call(k=3) == ps.PS_ERR_UNSUPPORTED
    assert call(Cout=257) == ps.PS_ERR_UNSUPPORTED
    assert call(x=MISALIGNED) == ps.PS_ERR_ALIGN


@fake_pointers
def test_post_process_validation(ps):
    lib = ps.lib()

    def pool(y=FAKE, b2=FAKE, out=FAKE, dtype=0, N=1, C=4, H=16, W=16, scale=2.0, k=4, s=0,
             p=0, d=1):
        return lib.ps_tanh_scale_bias_maxpool(y, b2, out, dtype, N, C, H, W, scale, k, s, p, d,
                                              None)

    assert pool(b2=None) == ps.PS_ERR_NULL
    assert pool(dtype=5) == ps.PS_ERR_PARAM
    assert pool(k=0) == ps.PS_ERR_PARAM
    assert pool(d=0) == ps.PS_ERR_PARAM
    assert pool(H=3, p=0) == ps.PS_ERR_SHAPE
    assert pool(out=MISALIGNED) == ps.PS_ERR_ALIGN

    def sm(y=FAKE, b2=FAKE, out=FAKE, N=1, C=128, H=8, W=8, scale=2.0):
        return lib.ps_softmax_bias_scale_sigmoid(y, b2, out, N, C, H, W, scale, None)

    assert sm(y=None) == ps.PS_ERR_NULL
    assert sm(C=0) == ps.PS_ERR_SHAPE
    assert sm(N=1 << 20, C=1 << 20) == ps.PS_ERR_SHAPE
    assert sm(y=MISALIGNED) == ps.PS_ERR_ALIGN


@fake_pointers
def test_convT_bf16_validation(ps):
    lib = ps.lib()

    def call(x=FAKE, w=FAKE, cb=None, b2=FAKE, y=FAKE, N=1, Cin=64, H=8, W=8, Cout=128, k=4,
             s=2, p=1, op=1, d=1, scale=2.0):
        return lib.ps_convT_softmax_bias_scale_sigmoid_bf16(x, w, cb, b2, y, N, Cin, H, W, Cout,
                                                            k, s, p, op, d, scale, None)

    assert call(b2=None) == ps.PS_ERR_NULL
    assert call(W=0) == ps.PS_ERR_SHAPE
    assert call(op=2) == ps.PS_ERR_PARAM
    assert call(s=3) == ps.PS_ERR_UNSUPPORTED
    assert call(Cout=48) == ps.PS_ERR_UNSUPPORTED       # not a multiple of 32
    assert call(Cin=80) == ps.PS_ERR_UNSUPPORTED        # weights exceed the LDS
    assert call(y=MISALIGNED) == ps.PS_ERR_ALIGN
