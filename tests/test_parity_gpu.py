"""Parity of the HIP kernels (through the C ABI) against the CPU oracle.

Every case prints its name, shape and seed before its first GPU call.  Sizes:
small cases the oracle finishes in well under a second, spanning several
tiles plus ragged tails, and the full workloads, every output element, in the
same launch configuration the benchmark times.

Bars: max-pool bit-exact (a -0/+0 tie is the one accepted difference, counted
and reported); fp32 conv paths abs 1e-4; bf16 paths abs 2e-2 and every output
the round-to-nearest-even of a value within the fp32 error budget of the
oracle's result; every output element written (NaN canary).
"""
import sys

import numpy as np
import pytest

import inputgen
import oracle
from cmp_util import assert_bf16_rne, assert_pool_bitexact, max_abs_err

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


def _dev(a, dev, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


def _canary(shape, dev, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device=dev)


# ----------------------------------------------------------------- maxpool ---
POOL_CASES = [
    # (N, C, H, W, k, s, p, d)
    (2, 3, 37, 45, 4, 1, 1, 1),     # stride-1 row kernel, ragged
    (1, 2, 70, 512, 4, 1, 1, 1),    # full-width strip, 3 bands
    (1, 2, 9, 700, 4, 1, 1, 1),     # two strips
    (2, 2, 33, 130, 3, 1, 1, 1),
    (1, 3, 20, 64, 2, 1, 0, 1),
    (1, 1, 40, 300, 5, 1, 2, 1),
    (1, 1, 40, 200, 7, 1, 3, 1),
    (1, 1, 19, 90, 8, 1, 0, 1),
    (1, 1, 5, 5, 4, 1, 3, 1),       # windows at the border only touch padding partly
    # bands of 32 output rows: the band below hands its first k-1 rows over through LDS
    (1, 3, 160, 96, 4, 1, 1, 1),    # 5 bands a plane: planes straddle workgroups
    (2, 1, 300, 70, 8, 1, 7, 1),    # k 8 with the largest padding, 10 bands
    (1, 5, 128, 40, 2, 1, 1, 1),    # k 2, a 1-row last band
    (1, 2, 97, 257, 6, 1, 5, 1),    # two strips, k 6
    (2, 2, 31, 29, 2, 2, 0, 1),     # direct kernel from here on
    (1, 2, 25, 27, 3, 2, 1, 1),
    (1, 1, 17, 21, 3, 1, 1, 2),
    (1, 1, 1, 1, 2, 1, 1, 2),       # all-padding window -> -inf
    (1, 2, 12, 14, 4, 4, 0, 1),
    (1, 2, 40, 50, 10, 3, 4, 1),    # window > 8: runtime-k kernel
    (1, 1, 33, 70, 3, 2, 1, 2),     # stride 2 and dilation 2
    (2, 3, 64, 64, 2, 2, 0, 1),
    (1, 1, 20, 300, 5, 3, 2, 1),
    (1, 2, 9, 9, 1, 1, 0, 1),       # k = 1: the identity
    (1, 1, 30, 31, 16, 5, 8, 1),
    (1, 2, 50, 45, 20, 3, 5, 1),    # windows beyond 16: runtime-k kernel
    (1, 1, 60, 60, 17, 2, 8, 2),    # k 17 dilated: a 33-wide window
    (1, 70000, 4, 4, 2, 2, 0, 1),   # more planes than one grid dimension holds
    # strided / dilated row-streaming kernel: several bands and strips
    (1, 2, 150, 600, 3, 2, 1, 1),   # k3 s2: 3 bands of 32 rows, 2 strips
    (1, 3, 140, 100, 3, 1, 2, 2),   # k3 s1 d2: 3 bands of 64 rows
    (2, 1, 70, 70, 4, 3, 3, 1),     # k4 s3, the largest padding
    (1, 1, 200, 40, 5, 2, 4, 2),    # k5 s2 d2: 4 bands
    (3, 2, 66, 520, 2, 1, 1, 2),    # k2 s1 d2: 3 strips, a ragged last strip
    # stride-1 row kernel, k <= 4 with every padding below k, rows of 260..1020
    # columns (one and two strips), several bands
    (1, 3, 100, 260, 2, 1, 0, 1),
    (2, 2, 70, 264, 2, 1, 1, 1),
    (1, 2, 66, 300, 3, 1, 0, 1),
    (1, 2, 66, 516, 3, 1, 1, 1),    # 1 KB rows
    (1, 1, 40, 1020, 3, 1, 2, 1),
    (2, 1, 70, 400, 4, 1, 0, 1),
    (1, 2, 35, 388, 4, 1, 2, 1),
    (1, 1, 96, 1016, 4, 1, 3, 1),
    (1, 5, 100, 512, 4, 1, 1, 1),   # 4 bands a plane: planes straddle workgroups
    # disjoint windows (stride = k in {2, 4}, no padding, even W): vector-load kernel
    (2, 3, 37, 50, 4, 4, 0, 1),     # unused last row and columns
    (1, 2, 130, 258, 2, 2, 0, 1),   # 3 column chunks, 17 row groups
    (1, 1, 4, 2, 2, 2, 0, 1),       # one column
]


@pytest.mark.parametrize("case", POOL_CASES)
def test_maxpool_small(dev, case):
    import pool_stencil_amd as ps
    N, C, H, W, k, s, p, d = case
    _say("maxpool", case, "seed 101")
    x = inputgen.randn(101, (N, C, H, W))
    ref = oracle.maxpool2d(x, k, s, p, d)
    xd = _dev(x, dev)
    import torch
    out = _canary(ref.shape, dev, torch.float32)
    ps.maxpool2d(xd, k, s, p, d, out=out)
    got = out.cpu().numpy()
    assert not np.isnan(got).any()
    assert_pool_bitexact(got, ref, f"maxpool {case}")


def test_maxpool_signed_zero_ties(dev):
    """Inputs full of +0 and -0 (and a few negatives): every output must equal the
    oracle's bit for bit, except that a window holding both zeros may give either
    sign; those ties are counted, and every other position stays bit-exact."""
    import pool_stencil_amd as ps
    import torch
    _say("maxpool signed zeros", "seed 102")
    x = inputgen.randn(102, (2, 3, 70, 90))
    sel = inputgen.uniform(103, x.shape, 0.0, 1.0)
    x = np.where(sel < 0.45, np.float32(0.0), np.where(sel < 0.9, np.float32(-0.0), -np.abs(x)))
    x = x.astype(np.float32)
    for (k, s, p, d) in [(4, 1, 1, 1), (3, 2, 1, 1), (3, 1, 2, 2), (5, 3, 2, 1)]:
        ref = oracle.maxpool2d(x, k, s, p, d)
        out = _canary(ref.shape, dev, torch.float32)
        ps.maxpool2d(_dev(x, dev), k, s, p, d, out=out)
        got = out.cpu().numpy()
        assert not np.isnan(got).any()
        assert_pool_bitexact(got, ref, f"maxpool signed zeros k{k} s{s} p{p} d{d}")


def test_maxpool_full_workload(dev):
    """The full 32x64x512x512 k4 s1 p1 d1 pool, every output compared bit for bit."""
    import pool_stencil_amd as ps
    import torch
    c = inputgen.workload("maxpool")
    _say("maxpool workload", c["x"].shape)
    ref = oracle.maxpool2d(c["x"], c["k"], c["stride"], c["pad"], c["dil"])
    xd = _dev(c["x"], dev)
    out = _canary(ref.shape, dev, torch.float32)
    ps.maxpool2d(xd, c["k"], c["stride"], c["pad"], c["dil"], out=out)
    got = out.cpu().numpy()
    del xd, out
    assert got.shape == (32, 64, 511, 511)
    assert not np.isnan(got).any()
    assert_pool_bitexact(got, ref, "maxpool workload")


@pytest.mark.parametrize("k,st,p,d,shape", [(3, 2, 1, 1, (32, 64, 256, 256)),
                                            (3, 1, 2, 2, (32, 64, 512, 512))])
def test_maxpool_general_full_workload(dev, k, st, p, d, shape):
    """The max-pool input under the downsampling (k3 s2 p1) and dilated (k3 s1 p2 d2)
    windows the benchmark times, every output compared bit for bit."""
    import pool_stencil_amd as ps
    import torch
    c = inputgen.workload("maxpool")
    _say("maxpool general workload", (k, st, p, d))
    ref = oracle.maxpool2d(c["x"], k, st, p, d)
    assert ref.shape == shape
    xd = _dev(c["x"], dev)
    out = _canary(ref.shape, dev, torch.float32)
    ps.maxpool2d(xd, k, st, p, d, out=out)
    got = out.cpu().numpy()
    del xd, out
    assert not np.isnan(got).any()
    assert_pool_bitexact(got, ref, f"maxpool workload k{k} s{st} p{p} d{d}")


# ------------------------------------------------------- fused conv + pool ---
def _run_conv(c, dev):
    import pool_stencil_amd as ps
    import torch
    if c["dtype"] == "bf16":
        xd = _dev(c["x_bits"].view(np.int16), dev).view(torch.bfloat16)
        wd = _dev(c["w_bits"].view(np.int16), dev).view(torch.bfloat16)
        odt = torch.bfloat16
    else:
        xd, wd, odt = _dev(c["x"], dev), _dev(c["w"], dev), torch.float32
    cb = None if c["conv_bias"] is None else _dev(c["conv_bias"], dev)
    b2 = _dev(c["bias2"], dev)
    shape = oracle.conv_pool_out_shape(c)
    out = _canary(shape, dev, odt)
    ps.conv_tanh_scale_bias_maxpool(xd, wd, cb, b2, c["scale"], c["pool_k"], c["pool_stride"],
                                    c["conv_stride"], c["conv_pad"], c["conv_dil"],
                                    c["pool_pad"], c["pool_dil"], out=out)
    return out.float().cpu().numpy()


CONV_CASES = [
    dict(N=2, Cin=8, H=32, W=32, Cout=16),                  # the tiny workload's shape
    dict(N=1, Cin=8, H=70, W=258, Cout=64),                 # 64-wide tiles, ragged tail
    dict(N=2, Cin=3, H=45, W=71, Cout=20),                  # Cin < 4, Cout ragged
    dict(N=1, Cin=5, H=30, W=40, Cout=130),                 # three 64-channel tiles
    dict(N=1, Cin=8, H=21, W=300, Cout=64, conv_pad=1),
    dict(N=1, Cin=8, H=19, W=33, Cout=32, conv_pad=2),
    dict(N=1, Cin=8, H=40, W=90, Cout=16, pool_k=2, pool_stride=2),
    dict(N=1, Cin=4, H=40, W=90, Cout=16, pool_k=3, pool_stride=3),
    dict(N=2, Cin=8, H=52, W=200, Cout=64, pool_k=3, pool_stride=3),  # 16-byte rows, k3
    dict(N=1, Cin=8, H=37, W=136, Cout=96, pool_k=3, pool_stride=3),  # 16-byte rows, 2 tiles
    dict(N=1, Cin=8, H=50, W=77, Cout=24, pool_k=5, pool_stride=5),
    dict(N=1, Cin=8, H=50, W=140, Cout=16, pool_k=6, pool_stride=6),
    dict(N=1, Cin=7, H=40, W=60, Cout=16, pool_k=7, pool_stride=7),
    dict(N=1, Cin=8, H=42, W=300, Cout=16, pool_k=8, pool_stride=8),
    dict(N=1, Cin=8, H=30, W=30, Cout=16, scale=-1.5),      # window minimum
    dict(N=1, Cin=8, H=30, W=30, Cout=16, scale=0.0),       # result is bias2
    dict(N=1, Cin=8, H=30, W=30, Cout=16, conv_bias=False),
    dict(N=1, Cin=1, H=6, W=6, Cout=1),                     # one pooled output
    # 16-byte rows (W % 8 == 0, no conv padding): the bf16 kernel stages the next rows
    # in LDS; 64 or 128 images give each persistent workgroup a run of several pooled
    # rows.  Pool 2..8 with one and two 16-column groups, several fill slices per
    # thread (pool 6 and 8), and more than 64 output channels.
    dict(N=64, Cin=8, H=66, W=32, Cout=16, pool_k=2, pool_stride=2),    # 1 group
    dict(N=64, Cin=8, H=34, W=64, Cout=24, pool_k=2, pool_stride=2),    # 2 groups
    dict(N=128, Cin=8, H=42, W=64, Cout=16, pool_k=5, pool_stride=5),   # 1 group
    dict(N=64, Cin=6, H=62, W=96, Cout=16, pool_k=5, pool_stride=5),    # 2 groups
    dict(N=64, Cin=8, H=74, W=96, Cout=16, pool_k=6, pool_stride=6),    # 2 slices/thread
    dict(N=32, Cin=8, H=98, W=264, Cout=16, pool_k=6, pool_stride=6),   # 2 groups, 2 slices
    dict(N=128, Cin=8, H=98, W=96, Cout=8, pool_k=8, pool_stride=8),    # 3 slices/thread
    dict(N=128, Cin=8, H=66, W=264, Cout=8, pool_k=8, pool_stride=8),   # 2 groups, 3 slices
    dict(N=128, Cin=8, H=34, W=96, Cout=130, pool_k=4, pool_stride=4),  # 3 channel tiles
    dict(N=64, Cin=8, H=30, W=64, Cout=96, pool_k=2, pool_stride=2),    # 2 channel tiles
    dict(N=128, Cin=8, H=64, W=128, Cout=16, pool_k=7, pool_stride=7),  # 2 groups
    # 16-byte rows, pool <= 4, one channel tile, 32 or 64 columns per strip: the bf16
    # kernel's 32x32x16 form (channel halves and column halves per wave), with ragged
    # channels and columns, Cin < 8, a window minimum, no conv bias and scale 0
    dict(N=16, Cin=5, H=36, W=128, Cout=40, pool_k=4, pool_stride=4),   # 31 columns
    dict(N=8, Cin=8, H=38, W=216, Cout=64, pool_k=4, pool_stride=4, scale=-0.7),  # 53
    dict(N=8, Cin=8, H=26, W=136, Cout=48, pool_k=3, pool_stride=3, conv_bias=False),
    dict(N=32, Cin=8, H=34, W=72, Cout=16, pool_k=2, pool_stride=2, scale=0.0),   # 35
    # the same form with runs of several pooled rows per workgroup (64 images, so each
    # plane splits into 8 runs): both ring phases and the row refill, for pool 2, 3, 4
    # and 32 or 64 columns per strip
    dict(N=64, Cin=8, H=50, W=72, Cout=16, pool_k=2, pool_stride=2),    # 3-row runs
    dict(N=64, Cin=8, H=86, W=136, Cout=24, pool_k=3, pool_stride=3, scale=-0.9),
    dict(N=64, Cin=8, H=82, W=128, Cout=32, pool_k=4, pool_stride=4),   # 31 columns
    dict(N=64, Cin=7, H=65, W=96, Cout=40, pool_k=3, pool_stride=3),    # 31 columns
]


@pytest.mark.parametrize("kw", CONV_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_pool_small(dev, kw, dtype):
    c = inputgen.random_conv_case(3000, dtype=dtype, **kw)
    _say("conv_pool", dtype, kw, "seed 3000")
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    got = _run_conv(c, dev)
    assert not np.isnan(got).any()
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    max_abs_err(got, ref, f"conv_pool {dtype} {kw}")
    np.testing.assert_allclose(got, ref, rtol=0, atol=tol)
    if dtype == "bf16":
        assert_bf16_rne(got, ref, f"conv_pool bf16 {kw}")


def test_conv_tiny_workload(dev):
    c = inputgen.workload("tiny_conv")
    _say("tiny_conv workload")
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    got = _run_conv(c, dev)
    assert got.shape == (2, 16, 7, 7)
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


@pytest.mark.parametrize("name,tol", [("conv", F32_TOL), ("conv_bf16", BF16_TOL)])
def test_conv_full_workload(dev, name, tol):
    """The full [128,8,256,256] workload, every one of the 32.5 M pooled outputs."""
    c = inputgen.workload(name)
    _say(name, "workload", c["x"].shape)
    got = _run_conv(c, dev)
    assert got.shape == (128, 64, 63, 63)
    assert not np.isnan(got).any()
    ref = oracle.conv_tanh_scale_bias_maxpool(c)
    max_abs_err(got, ref, f"{name} workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=tol)
    if name == "conv_bf16":
        assert_bf16_rne(got, ref, "conv_bf16 workload")


# ------------------------------------------------ convT + channel softmax ---
def _run_convT(c, dev):
    import pool_stencil_amd as ps
    import torch
    if c["dtype"] == "bf16":
        xd = _dev(c["x_bits"].view(np.int16), dev).view(torch.bfloat16)
        wd = _dev(c["w_bits"].view(np.int16), dev).view(torch.bfloat16)
    else:
        xd, wd = _dev(c["x"], dev), _dev(c["w"], dev)
    cb = None if c["convT_bias"] is None else _dev(c["convT_bias"], dev)
    b2 = _dev(c["bias2"], dev)
    out = _canary(oracle.convT_out_shape(c), dev, xd.dtype)
    ps.convT_softmax_bias_scale_sigmoid(xd, wd, cb, b2, c["scale"], c["stride"], c["pad"],
                                        c["output_padding"], c["dil"], out=out)
    return out.float().cpu().numpy()


CONVT_CASES = [
    dict(N=2, Cin=64, H=9, W=7, Cout=128),
    dict(N=1, Cin=64, H=16, W=16, Cout=128, output_padding=0),
    dict(N=3, Cin=13, H=5, W=11, Cout=48),
    dict(N=1, Cin=4, H=3, W=3, Cout=16),
    dict(N=1, Cin=1, H=1, W=1, Cout=16),
    dict(N=2, Cin=64, H=8, W=8, Cout=128, scale=-0.5, convT_bias=False),
    dict(N=1, Cin=32, H=12, W=20, Cout=112),
    dict(N=1, Cin=70, H=6, W=70, Cout=128),       # Cin not a multiple of 4, 150 KB of weights
    dict(N=4, Cin=7, H=13, W=9, Cout=64, output_padding=0),  # channels past Cin, last image
    # any padding: the class -> kernel tap / input offset mapping moves with its parity
    dict(N=2, Cin=16, H=9, W=11, Cout=64, pad=0),
    dict(N=1, Cin=16, H=10, W=7, Cout=32, pad=0, output_padding=0),
    dict(N=2, Cin=20, H=9, W=12, Cout=48, pad=2),
    dict(N=1, Cin=64, H=8, W=9, Cout=128, pad=3, output_padding=0),
    dict(N=1, Cin=8, H=12, W=10, Cout=16, pad=5),
    dict(N=1, Cin=4, H=3, W=3, Cout=16, pad=3),               # 1x1 .. output rows
    # more than 128 channels: one 16-pixel group per wave tile
    dict(N=2, Cin=64, H=7, W=9, Cout=144),
    dict(N=1, Cin=36, H=6, W=10, Cout=256),                   # the largest weight tile
    dict(N=1, Cin=20, H=5, W=7, Cout=240, pad=2, scale=-0.7),
    dict(N=3, Cin=9, H=4, W=6, Cout=176, pad=0, convT_bias=False),
    # Cout not a multiple of 16: the last channel tile masked out of the softmax and
    # the stores
    dict(N=2, Cin=16, H=7, W=9, Cout=100),
    dict(N=1, Cin=8, H=5, W=6, Cout=1),                       # softmax of one channel
    dict(N=1, Cin=20, H=6, W=7, Cout=250, pad=0),
    dict(N=3, Cin=9, H=4, W=5, Cout=37, scale=-0.8, convT_bias=False),
]


# the row-class kernel: Cout 128, Cin <= 64, W a multiple of 4, >= 64 column
# positions per output row (segments of a plane per workgroup when there are fewer
# planes than CUs, so several cases start mid-plane; N = 64 gives units of several
# tiles, the steady-state row ring)
CONVT_ROWS_CASES = [
    dict(N=2, Cin=64, H=5, W=64, Cout=128),
    dict(N=1, Cin=64, H=7, W=64, Cout=128, output_padding=0),
    dict(N=3, Cin=20, H=4, W=68, Cout=128, pad=0),
    dict(N=2, Cin=37, H=5, W=72, Cout=128, pad=2, scale=-0.6, convT_bias=False),
    dict(N=1, Cin=64, H=6, W=76, Cout=128, pad=3, output_padding=0),
    dict(N=1, Cin=16, H=9, W=84, Cout=128),
    dict(N=1, Cin=8, H=6, W=68, Cout=128, pad=5),
    dict(N=64, Cin=64, H=6, W=64, Cout=128),
    # a plane's last tile of at most 16 positions runs one position block's matrix work:
    # last tiles of 16 and 15 positions (one block), then 17 and 16
    dict(N=1, Cin=32, H=15, W=64, Cout=128),
    dict(N=1, Cin=32, H=16, W=64, Cout=128, scale=-0.9),
]
CONVT_CASES += CONVT_ROWS_CASES


@pytest.mark.parametrize("kw", CONVT_CASES)
def test_convT_small(dev, kw):
    c = inputgen.random_convT_case(4000, **kw)
    _say("convT", kw, "seed 4000")
    ref = oracle.convT_softmax_bias_scale_sigmoid(c)
    got = _run_convT(c, dev)
    assert not np.isnan(got).any()
    max_abs_err(got, ref, f"convT {kw}")
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


CONVT_BF16_CASES = [
    dict(N=2, Cin=64, H=9, W=7, Cout=128),
    dict(N=1, Cin=64, H=16, W=16, Cout=128, output_padding=0),
    dict(N=3, Cin=13, H=5, W=11, Cout=64),
    dict(N=1, Cin=4, H=3, W=3, Cout=32),
    dict(N=1, Cin=1, H=1, W=1, Cout=32),
    dict(N=2, Cin=64, H=8, W=8, Cout=128, scale=-0.5, convT_bias=False),
    dict(N=1, Cin=32, H=12, W=20, Cout=96),
    dict(N=1, Cin=70, H=6, W=70, Cout=128),       # Cin not a multiple of 4; 3 column blocks
    # W a multiple of 8: the LDS-staged kernel (the 16- and 8-wide cases above too)
    dict(N=2, Cin=13, H=5, W=8, Cout=32),         # one ragged channel chunk
    dict(N=1, Cin=20, H=7, W=16, Cout=96, output_padding=0),
    dict(N=3, Cin=64, H=9, W=24, Cout=128),       # items end mid-row, three images
    dict(N=1, Cin=8, H=1, W=8, Cout=64),          # one input row
    dict(N=2, Cin=64, H=4, W=64, Cout=128, scale=-0.5),
    dict(N=1, Cin=32, H=3, W=160, Cout=64),       # rows longer than a work item
    dict(N=1, Cin=16, H=2, W=256, Cout=32, output_padding=0),
    # any padding, both kernels (W % 8 == 0 takes the staged one)
    dict(N=2, Cin=16, H=9, W=16, Cout=64, pad=0),             # positions up to column W + 1
    dict(N=1, Cin=16, H=7, W=8, Cout=32, pad=0, output_padding=0),
    dict(N=2, Cin=24, H=6, W=24, Cout=96, pad=2),
    dict(N=1, Cin=64, H=5, W=16, Cout=128, pad=3, output_padding=0),
    dict(N=1, Cin=8, H=12, W=40, Cout=32, pad=5),
    dict(N=2, Cin=16, H=9, W=11, Cout=64, pad=0),             # the pixel-tile kernel
    dict(N=1, Cin=20, H=7, W=13, Cout=96, pad=2),
    dict(N=1, Cin=13, H=6, W=9, Cout=32, pad=3, output_padding=0),
]


# the bf16 row-class kernel: Cout 128, Cin <= 64, W a multiple of 8, >= 64 column
# positions per output row
CONVT_BF16_ROWS_CASES = [
    dict(N=2, Cin=64, H=5, W=64, Cout=128),
    dict(N=1, Cin=64, H=6, W=64, Cout=128, output_padding=0),
    dict(N=3, Cin=24, H=4, W=72, Cout=128, pad=0),
    dict(N=2, Cin=40, H=5, W=80, Cout=128, pad=2, scale=-0.6, convT_bias=False),
    dict(N=1, Cin=64, H=6, W=72, Cout=128, pad=3, output_padding=0),
    dict(N=1, Cin=8, H=6, W=72, Cout=128, pad=5),
    dict(N=64, Cin=64, H=6, W=64, Cout=128),
]
CONVT_BF16_CASES += CONVT_BF16_ROWS_CASES


@pytest.mark.parametrize("kw", CONVT_BF16_CASES)
def test_convT_bf16_small(dev, kw):
    """bf16 x/w/output: the oracle runs the fp32 definition on the bf16-rounded inputs;
    bar abs 2e-2 (outputs lie in (0, 1), where one bf16 ulp is at most 2^-8)."""
    c = inputgen.random_convT_case(4100, dtype="bf16", **kw)
    _say("convT bf16", kw, "seed 4100")
    ref = oracle.convT_softmax_bias_scale_sigmoid(c)
    got = _run_convT(c, dev)
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, ref, rtol=0, atol=BF16_TOL)
    assert_bf16_rne(got, ref, f"convT bf16 {kw}")


def _softmax_invariant(got, c, atol):
    """From the outputs alone: sum_c (logit(y_c)/scale - bias2_c) == 1 on every pixel."""
    g = got.astype(np.float64)
    sm = np.log(g / (1.0 - g)) / c["scale"] - c["bias2"].astype(np.float64).reshape(1, -1, 1, 1)
    np.testing.assert_allclose(sm.sum(axis=1), 1.0, atol=atol)


def test_convT_full_workload(dev):
    """The full [128,64,64,64] -> [128,128,129,129] workload, every output element."""
    c = inputgen.workload("convT")
    _say("convT workload", c["x"].shape)
    got = _run_convT(c, dev)
    assert got.shape == (128, 128, 129, 129)
    assert not np.isnan(got).any()
    _softmax_invariant(got[:4], c, 5e-3)
    ref = oracle.convT_softmax_bias_scale_sigmoid(c)
    max_abs_err(got, ref, "convT workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=F32_TOL)


def test_convT_bf16_full_workload(dev):
    c = inputgen.workload("convT_bf16")
    _say("convT_bf16 workload", c["x"].shape)
    got = _run_convT(c, dev)
    assert got.shape == (128, 128, 129, 129)
    assert not np.isnan(got).any()
    ref = oracle.convT_softmax_bias_scale_sigmoid(c)
    max_abs_err(got, ref, "convT_bf16 workload")
    np.testing.assert_allclose(got, ref, rtol=0, atol=BF16_TOL)
    assert_bf16_rne(got, ref, "convT_bf16 workload")
