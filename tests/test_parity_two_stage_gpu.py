"""Parity of the unfused pipelines' stages (through the C ABI) against the oracle.

Covers ps_convT2d (the transposed conv without its epilogue), the two
post-processing entry points on stored outputs, and both two-stage pipelines
end to end against the fused oracle, at small sizes and at the full workload
sizes (every output element).  Each case prints its name and shape before its
first GPU call.

Bars: fp32 abs 1e-4; bf16 stored conv outputs abs 2e-2 (the outputs of the
epilogue are bounded by |scale| + |bias2|) and round-to-nearest-even of a value
within the fp32 error budget of the oracle's result; every output written (NaN
canary); windows lying wholly in the padding give -inf on both sides.
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


def _nan(shape, dev, dtype=None):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype or torch.float32, device=dev)


# ------------------------------------------------------ plain transposed conv ---
CONVT2D_CASES = [
    dict(N=2, Cin=64, H=9, W=7, Cout=128),
    dict(N=1, Cin=13, H=5, W=11, Cout=48, output_padding=0),
    dict(N=1, Cin=1, H=1, W=1, Cout=16),
    dict(N=2, Cin=32, H=8, W=8, Cout=112, convT_bias=False),
    dict(N=1, Cin=16, H=6, W=9, Cout=64, pad=0),
    dict(N=1, Cin=12, H=7, W=6, Cout=48, pad=3, output_padding=0),
    dict(N=1, Cin=32, H=5, W=6, Cout=256),
    dict(N=2, Cin=12, H=6, W=5, Cout=37),                     # Cout not a multiple of 16
    dict(N=1, Cin=4, H=3, W=4, Cout=3, pad=0, output_padding=0),
    # the row-class kernel without its softmax epilogue
    dict(N=2, Cin=64, H=5, W=64, Cout=128),
    dict(N=1, Cin=24, H=6, W=72, Cout=128, pad=2, output_padding=0, convT_bias=False),
]


@pytest.mark.parametrize("kw", CONVT2D_CASES)
def test_convT2d_small(dev, kw):
    import pool_stencil_amd as ps
    c = inputgen.random_convT_case(7000, **kw)
    _say("convT2d", kw, "seed 7000")
    ref = oracle.conv_transpose2d(c["x"], c["w"], c["convT_bias"], c["stride"], c["pad"],
                                  c["output_padding"], c["dil"])
    cb = None if c["convT_bias"] is None else _dev(c["convT_bias"], dev)
    out = _nan(ref.shape, dev)
    ps.convT2d(_dev(c["x"], dev), _dev(c["w"], dev), cb, c["stride"], c["pad"],
               c["output_padding"], c["dil"], out=out)
    got = out.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


# ------------------------------------------ epilogue + pool of a stored conv ---
POOL_EPI_CASES = [
    # (N, C, H, W, k, stride, pad, dil, scale)
    (2, 5, 38, 41, 4, 4, 0, 1, 2.0),
    (1, 3, 30, 33, 3, 2, 1, 1, 2.0),
    (1, 4, 25, 27, 2, 1, 0, 2, -1.5),
    (1, 2, 20, 20, 3, 3, 1, 1, 0.0),
    (1, 3, 17, 300, 5, 1, 2, 1, 0.7),
    (1, 2, 6, 6, 2, 1, 2, 1, 2.0),      # windows wholly in the padding -> -inf
    (1, 3, 150, 140, 4, 4, 1, 1, -0.6),  # row-streaming kernel: 5 bands, padding, scale < 0
    (1, 2, 70, 600, 3, 2, 1, 1, 1.3),   # 256-column strips, a ragged second strip
    # disjoint windows, even W: the vector-load kernel (fp32)
    (2, 5, 38, 42, 4, 4, 0, 1, -1.3),
    (1, 3, 66, 130, 2, 2, 0, 1, 0.0),
    (1, 64, 254, 254, 4, 4, 0, 1, 2.0),  # one image of the conv workload's stored output
]


@pytest.mark.parametrize("case", POOL_EPI_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tanh_scale_bias_maxpool_small(dev, case, dtype):
    import pool_stencil_amd as ps
    import torch
    N, C, H, W, k, s, p, d, scale = case
    _say("tanh_scale_bias_maxpool", dtype, case, "seed 7100")
    y = inputgen.randn(7100, (N, C, H, W), 2.0)
    b2 = inputgen.randn(7101, (C,), 0.1)
    if dtype == "bf16":
        bits = inputgen.to_bf16_bits(y)
        y = inputgen.bf16_bits_to_f32(bits).reshape(y.shape)
        yd = _dev(bits.view(np.int16).reshape(y.shape), dev).view(torch.bfloat16)
    else:
        yd = _dev(y, dev)
    ref = oracle.tanh_scale_bias_maxpool(y, b2, scale, k, s, p, d)
    out = _nan(ref.shape, dev, yd.dtype)
    ps.tanh_scale_bias_maxpool(yd, _dev(b2, dev), scale, k, s, p, d, out=out)
    got = out.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    max_abs_err(got, ref, f"tanh_scale_bias_maxpool {dtype} {case}")
    np.testing.assert_allclose(got[fin], ref[fin], rtol=0,
                               atol=BF16_TOL if dtype == "bf16" else F32_TOL)
    if dtype == "bf16":
        assert_bf16_rne(got, ref, f"tanh_scale_bias_maxpool bf16 {case}")


# ------------------------------------------- softmax post-process of a convT ---
@pytest.mark.parametrize("C,H,W", [(8, 9, 13), (48, 9, 13), (128, 9, 13), (130, 9, 13),
                                   (200, 9, 13), (128, 17, 19), (128, 16, 16)])
@pytest.mark.parametrize("inplace", [False, True])
def test_softmax_bias_scale_sigmoid_small(dev, C, H, W, inplace):
    """Channel counts up to 128 keep a pixel's channels in registers, more take two
    passes; the 128-channel shapes cover one, several and ragged 256-pixel blocks."""
    import pool_stencil_amd as ps
    _say("softmax_bias_scale_sigmoid", C, H, W, "inplace" if inplace else "", "seed 7200")
    y = inputgen.randn(7200, (2, C, H, W), 3.0)
    b2 = inputgen.randn(7201, (C,), 0.1)
    ref = oracle.softmax_bias_scale_sigmoid(y, b2, -0.8)
    yd = _dev(y, dev)
    out = yd if inplace else _nan(y.shape, dev)
    ps.softmax_bias_scale_sigmoid(yd, _dev(b2, dev), -0.8, out=out)
    got = out.cpu().numpy()
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


# ------------------------------------------------------ two-stage pipelines ---
def test_two_stage_conv_small(dev):
    """conv to memory (ps_conv2d), then epilogue + pool of the stored output, against the
    fused oracle."""
    import pool_stencil_amd as ps
    c = inputgen.random_conv_case(7300, N=2, Cin=8, H=40, W=44, Cout=64)
    _say("two-stage conv", "seed 7300")
    y = ps.conv2d(_dev(c["x"], dev), _dev(c["w"], dev), _dev(c["conv_bias"], dev))
    out = ps.tanh_scale_bias_maxpool(y, _dev(c["bias2"], dev), c["scale"], c["pool_k"])
    np.testing.assert_allclose(out.cpu().numpy(), oracle.conv_tanh_scale_bias_maxpool(c), rtol=0,
                               atol=F32_TOL)


def test_two_stage_convT_small(dev):
    """convT to memory (ps_convT2d), then the softmax post-process in place, against the
    fused oracle."""
    import pool_stencil_amd as ps
    c = inputgen.random_convT_case(7400, N=2, Cin=64, H=9, W=10, Cout=128)
    _say("two-stage convT", "seed 7400")
    y = ps.convT2d(_dev(c["x"], dev), _dev(c["w"], dev), _dev(c["convT_bias"], dev))
    ps.softmax_bias_scale_sigmoid(y, _dev(c["bias2"], dev), c["scale"], out=y)
    np.testing.assert_allclose(y.cpu().numpy(), oracle.convT_softmax_bias_scale_sigmoid(c),
                               rtol=0, atol=F32_TOL)


def test_two_stage_conv_workload(dev):
    """The conv workload through the unfused pipeline (the 2.1 GB conv output stored),
    every pooled output against the fused oracle."""
    import pool_stencil_amd as ps
    c = inputgen.workload("conv")
    _say("two-stage conv workload", c["x"].shape)
    y = ps.conv2d(_dev(c["x"], dev), _dev(c["w"], dev), _dev(c["conv_bias"], dev))
    assert tuple(y.shape) == (128, 64, 254, 254)
    out = ps.tanh_scale_bias_maxpool(y, _dev(c["bias2"], dev), c["scale"], c["pool_k"])
    del y
    got = out.cpu().numpy()
    assert got.shape == (128, 64, 63, 63)
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    max_abs_err(got, ref, "two-stage conv workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


def test_two_stage_convT_workload(dev):
    """The convT workload through the unfused pipeline (1.09 GB stored, post-processed
    in place), every output against the fused oracle."""
    import pool_stencil_amd as ps
    c = inputgen.workload("convT")
    _say("two-stage convT workload", c["x"].shape)
    y = ps.convT2d(_dev(c["x"], dev), _dev(c["w"], dev), _dev(c["convT_bias"], dev))
    ps.softmax_bias_scale_sigmoid(y, _dev(c["bias2"], dev), c["scale"], out=y)
    got = y.cpu().numpy()
    del y
    assert got.shape == (128, 128, 129, 129)
    ref = oracle.convT_softmax_bias_scale_sigmoid(c)
    max_abs_err(got, ref, "two-stage convT workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)
