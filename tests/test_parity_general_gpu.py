"""Parity of the general conv kernel (through the C ABI) against the CPU oracle.

Covers the fused conv + pool beyond the 3x3 / few-channel / disjoint-window
case (any kernel, stride, padding, dilation, channel count; overlapping,
padded and dilated pools) and the plain Conv2d entry point.  Each case prints
its name and shape before its first GPU call.

Bars: fused fp32 abs 1e-4, fused bf16 abs 2e-2 (outputs are bounded by
|scale| + |bias2|); plain conv fp32 abs 1e-4; plain conv bf16: the fp32 sum
rounded once to bf16, so |got - ref| <= 2^-8 |ref| + 1e-4.  Every bf16 output
is also the round-to-nearest-even of a value within the fp32 error budget of
the oracle's result.  The full-size workload is compared element by element.
A NaN canary checks that every output element is written; windows lying wholly
in the pool's padding must give -inf on both sides.
"""
import sys

import numpy as np
import pytest

import inputgen
import oracle
from cmp_util import assert_bf16_rne, max_abs_err

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pool_stencil_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _inputs(c, dev):
    import torch
    if c["dtype"] == "bf16":
        xd = _dev(c["x_bits"].view(np.int16), dev).view(torch.bfloat16)
        wd = _dev(c["w_bits"].view(np.int16), dev).view(torch.bfloat16)
    else:
        xd, wd = _dev(c["x"], dev), _dev(c["w"], dev)
    cb = None if c["conv_bias"] is None else _dev(c["conv_bias"], dev)
    return xd, wd, cb


def _run_fused(c, dev):
    import pool_stencil_amd as ps
    import torch
    xd, wd, cb = _inputs(c, dev)
    b2 = _dev(c["bias2"], dev)
    out = torch.full(oracle.conv_pool_out_shape(c), float("nan"), dtype=xd.dtype, device=dev)
    ps.conv_tanh_scale_bias_maxpool(xd, wd, cb, b2, c["scale"], c["pool_k"], c["pool_stride"],
                                    c["conv_stride"], c["conv_pad"], c["conv_dil"],
                                    c["pool_pad"], c["pool_dil"], out=out)
    return out.float().cpu().numpy()


GENERAL_CASES = [
    dict(N=1, Cin=16, H=30, W=40, Cout=32, pool_k=2, pool_stride=2),          # Cin > 8
    dict(N=2, Cin=64, H=20, W=36, Cout=128, conv_pad=1, pool_k=3, pool_stride=2,
         pool_pad=1),                                                          # overlapping pool
    dict(N=1, Cin=37, H=18, W=23, Cout=70, conv_pad=1, pool_k=2, pool_stride=2),  # ragged chunk/Cout
    dict(N=1, Cin=8, H=33, W=47, Cout=16, conv_stride=2, pool_k=2, pool_stride=2),  # conv stride 2
    dict(N=1, Cin=4, H=30, W=30, Cout=16, conv_dil=2, pool_k=3, pool_stride=2),     # conv dilation 2
    dict(N=1, Cin=3, H=26, W=31, Cout=24, kH=5, kW=5, conv_pad=2, pool_k=3, pool_stride=1,
         pool_pad=1),                                                          # 5x5, stride-1 pool
    dict(N=1, Cin=32, H=20, W=20, Cout=16, kH=1, kW=1, pool_k=2, pool_stride=2),    # 1x1 conv
    dict(N=1, Cin=3, H=40, W=44, Cout=64, kH=7, kW=7, conv_stride=2, conv_pad=3, pool_k=3,
         pool_stride=2, pool_pad=1),                                           # 7x7 s2 stem
    dict(N=1, Cin=8, H=25, W=29, Cout=16, kH=3, kW=5, conv_pad=1, pool_k=2, pool_stride=2),
    dict(N=1, Cin=8, H=30, W=30, Cout=16, pool_k=3, pool_stride=1, pool_pad=2, pool_dil=2),
    dict(N=1, Cin=8, H=12, W=12, Cout=16, pool_k=2, pool_stride=1, pool_pad=2),  # -inf windows
    dict(N=1, Cin=16, H=24, W=24, Cout=16, conv_pad=1, pool_k=3, pool_stride=2, scale=-1.5),
    dict(N=1, Cin=16, H=24, W=24, Cout=16, conv_pad=1, pool_k=3, pool_stride=2, scale=0.0),
    dict(N=1, Cin=130, H=10, W=12, Cout=16, pool_k=2, pool_stride=2),          # 9 channel chunks
    dict(N=1, Cin=8, H=30, W=30, Cout=16, conv_pad=3, pool_k=2, pool_stride=2),  # conv pad 3
    dict(N=1, Cin=8, H=40, W=300, Cout=16, pool_k=10, pool_stride=10),         # pool window 10
    dict(N=1, Cin=2, H=9, W=9, Cout=3, conv_dil=3, pool_k=1, pool_stride=1),   # 1x1 pool
    dict(N=1, Cin=8, H=30, W=30, Cout=16, conv_bias=False, pool_k=3, pool_stride=3,
         pool_pad=1),
    dict(N=3, Cin=12, H=70, W=90, Cout=48, conv_pad=1, pool_k=2, pool_stride=1),  # many tiles
    dict(N=2, Cin=20, H=26, W=30, Cout=72, conv_pad=1, pool_k=3, pool_stride=2,
         pool_pad=1),                                                           # partial chunk, 2 images
]


@pytest.mark.parametrize("kw", GENERAL_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_general_fused_small(dev, kw, dtype):
    c = inputgen.random_conv_case(5000, dtype=dtype, **kw)
    _say("conv_general", dtype, kw, "seed 5000")
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    got = _run_fused(c, dev)
    assert got.shape == ref.shape
    assert not np.isnan(got).any()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    fin = np.isfinite(ref)
    max_abs_err(got, ref, f"conv_general {dtype} {kw}")
    np.testing.assert_allclose(got[fin], ref[fin], rtol=0, atol=tol)
    if dtype == "bf16":
        assert_bf16_rne(got, ref, f"conv_general bf16 {kw}")


def test_general_fused_workload(dev):
    """The 32x64x128x128 -> 128-channel 3x3 conv + 3x3/2 pool at full size, every one
    of the 16.8 M pooled outputs."""
    c = inputgen.workload("conv_general")
    _say("conv_general workload", c["x"].shape)
    got = _run_fused(c, dev)
    assert got.shape == (32, 128, 64, 64)
    assert not np.isnan(got).any()
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    max_abs_err(got, ref, "conv_general workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


# ------------------------------------------------------------- plain conv ---
CONV2D_CASES = [
    dict(N=2, Cin=8, H=34, W=35, Cout=64),
    dict(N=1, Cin=64, H=20, W=21, Cout=128, conv_pad=1),
    dict(N=1, Cin=3, H=40, W=41, Cout=64, kH=7, kW=7, conv_stride=2, conv_pad=3),
    dict(N=1, Cin=13, H=17, W=19, Cout=20, kH=3, kW=5, conv_stride=2, conv_pad=1, conv_dil=2),
    dict(N=1, Cin=16, H=15, W=15, Cout=16, kH=1, kW=1),
    dict(N=1, Cin=5, H=3, W=3, Cout=7),                                        # one output pixel
    dict(N=1, Cin=8, H=24, W=24, Cout=16, conv_bias=False),
]


@pytest.mark.parametrize("kw", CONV2D_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv2d_small(dev, kw, dtype):
    import pool_stencil_amd as ps
    import torch
    c = inputgen.random_conv_case(6000, dtype=dtype, **kw)
    _say("conv2d", dtype, kw, "seed 6000")
    ref = oracle.conv2d(c["x"], c["w"], c["conv_bias"], c["conv_stride"], c["conv_pad"],
                        c["conv_dil"])
    xd, wd, cb = _inputs(c, dev)
    out = torch.full(ref.shape, float("nan"), dtype=xd.dtype, device=dev)
    ps.conv2d(xd, wd, cb, c["conv_stride"], c["conv_pad"], c["conv_dil"], out=out)
    got = out.float().cpu().numpy()
    assert not np.isnan(got).any()
    if dtype == "bf16":
        np.testing.assert_allclose(got, ref, rtol=2.0 ** -8, atol=1e-4)
        assert_bf16_rne(got, ref, f"conv2d bf16 {kw}")
    else:
        max_abs_err(got, ref, f"conv2d {kw}")
        np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)
