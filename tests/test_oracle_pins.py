"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, zero instead of -inf padding, a
flipped kernel, a wrong epilogue order) fails at least one of them:

  * closed-form output extents printed on the pages (tests/golden/shapes.txt);
  * the convT row -> tap table printed on the l2_p91 page
    (tests/golden/convT_phase_taps.txt);
  * library routines the operation reduces to: torch's CPU conv2d,
    conv_transpose2d, max_pool2d and softmax in float64;
  * independent numpy formulations (sliding windows, im2col, zero insertion);
  * identities and invariants: no kernel flip (one-hot input), linearity,
    the convT / conv adjoint identity, the monotone reorder of max and the
    epilogue, the separable max, softmax summing to one and shift invariance.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import inputgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------- shapes ---
def _golden_shapes():
    rows = []
    with open(os.path.join(GOLDEN, "shapes.txt")) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if not line or line.startswith("#"):
                continue
            op, n, k, s, p, d, opad, out = line.split()
            rows.append((op, int(n), int(k), int(s), int(p), int(d), int(opad), int(out)))
    return rows


@pytest.mark.parametrize("row", _golden_shapes())
def test_printed_output_extents(row):
    op, n, k, s, p, d, opad, out = row
    if op in ("conv", "pool"):
        assert oracle.window_out_dim(n, k, s, p, d) == out
    else:
        assert oracle.convT_out_dim(n, k, s, p, opad, d) == out


def test_window_that_does_not_fit_has_no_output():
    assert oracle.window_out_dim(2, 3, 1, 0, 1) <= 0
    assert oracle.window_out_dim(2, 2, 1, 0, 2) <= 0
    assert oracle.window_out_dim(3, 2, 1, 0, 2) == 1


# ------------------------------------------------------------------ conv2d ---
@pytest.mark.parametrize("cfg", [
    dict(N=2, Cin=3, H=9, W=11, Cout=4, k=3, s=1, p=0, d=1),
    dict(N=1, Cin=5, H=12, W=7, Cout=3, k=3, s=2, p=1, d=1),
    dict(N=2, Cin=2, H=13, W=13, Cout=2, k=3, s=1, p=2, d=2),
    dict(N=1, Cin=4, H=8, W=10, Cout=5, k=2, s=3, p=1, d=1),
])
def test_conv2d_matches_torch_float64(cfg):
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, (cfg["N"], cfg["Cin"], cfg["H"], cfg["W"])).astype(np.float32)
    w = rng.uniform(-1, 1, (cfg["Cout"], cfg["Cin"], cfg["k"], cfg["k"])).astype(np.float32)
    b = rng.uniform(-1, 1, cfg["Cout"]).astype(np.float32)
    got = oracle.conv2d(x, w, b, cfg["s"], cfg["p"], cfg["d"])
    ref = F.conv2d(_t(x), _t(w), _t(b), stride=cfg["s"], padding=cfg["p"], dilation=cfg["d"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_conv2d_no_kernel_flip_one_hot():
    """A one-hot input at (ci, i, j) must reproduce w[co, ci, kh, kw] at y[co, i-kh, j-kw]
    (cross-correlation, as nn.Conv2d computes); a flipped kernel fails this."""
    rng = np.random.default_rng(2)
    Cin, Cout, H, W = 3, 2, 7, 8
    w = rng.uniform(-1, 1, (Cout, Cin, 3, 3)).astype(np.float32)
    ci, i, j = 1, 4, 5
    x = np.zeros((1, Cin, H, W), np.float32)
    x[0, ci, i, j] = 1.0
    y = oracle.conv2d(x, w)
    for co in range(Cout):
        for kh in range(3):
            for kw in range(3):
                assert y[0, co, i - kh, j - kw] == w[co, ci, kh, kw]
    assert np.count_nonzero(y) == np.count_nonzero(w[:, ci])


def test_conv2d_im2col_numpy():
    """An independent im2col formulation: y = W_flat @ patches + b."""
    rng = np.random.default_rng(3)
    N, Cin, H, W, Cout = 2, 4, 6, 9, 5
    x = rng.uniform(-1, 1, (N, Cin, H, W)).astype(np.float32)
    w = rng.uniform(-1, 1, (Cout, Cin, 3, 3)).astype(np.float32)
    b = rng.uniform(-1, 1, Cout).astype(np.float32)
    win = np.lib.stride_tricks.sliding_window_view(x.astype(np.float64), (3, 3), axis=(2, 3))
    # win [N, Cin, OH, OW, 3, 3] -> [N, OH, OW, Cin*9]
    patches = win.transpose(0, 2, 3, 1, 4, 5).reshape(N, H - 2, W - 2, Cin * 9)
    ref = patches @ w.reshape(Cout, -1).astype(np.float64).T + b
    np.testing.assert_allclose(oracle.conv2d(x, w, b), ref.transpose(0, 3, 1, 2), atol=1e-12)


def test_conv2d_1x1_is_channel_matmul_and_linear():
    rng = np.random.default_rng(4)
    x = rng.uniform(-1, 1, (1, 6, 5, 4)).astype(np.float32)
    w = rng.uniform(-1, 1, (3, 6, 1, 1)).astype(np.float32)
    ref = np.einsum("oc,nchw->nohw", w[:, :, 0, 0].astype(np.float64), x.astype(np.float64))
    np.testing.assert_allclose(oracle.conv2d(x, w), ref, atol=1e-12)
    w3 = rng.uniform(-1, 1, (3, 6, 3, 3)).astype(np.float32)
    x2 = rng.uniform(-1, 1, x.shape).astype(np.float32)
    lhs = oracle.conv2d(x, w3) + oracle.conv2d(x2, w3)
    rhs = oracle.conv2d(x.astype(np.float64) + x2, w3)  # float64 sum, re-rounded to float32
    np.testing.assert_allclose(lhs, rhs, atol=1e-6)


# ----------------------------------------------------------------- maxpool ---
def _numpy_maxpool(x, k, s, p, d):
    xp = np.pad(x.astype(np.float64), ((0, 0), (0, 0), (p, p), (p, p)), constant_values=-np.inf)
    N, C, Hp, Wp = xp.shape
    OH = (Hp - d * (k - 1) - 1) // s + 1
    OW = (Wp - d * (k - 1) - 1) // s + 1
    out = np.full((N, C, OH, OW), -np.inf)
    for a in range(k):
        for b in range(k):
            sl = xp[:, :, a * d: a * d + s * (OH - 1) + 1: s, b * d: b * d + s * (OW - 1) + 1: s]
            out = np.maximum(out, sl)
    return out


@pytest.mark.parametrize("k,s,p,d", [(4, 1, 1, 1), (2, 2, 0, 1), (3, 2, 1, 1), (3, 1, 1, 2),
                                     (4, 4, 0, 1), (1, 1, 0, 1), (5, 3, 2, 1)])
def test_maxpool_matches_numpy_and_torch(k, s, p, d):
    x = inputgen.randn(77, (2, 3, 13, 17))
    got = oracle.maxpool2d(x, k, s, p, d)
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got.astype(np.float64), _numpy_maxpool(x, k, s, p, d))
    ref = F.max_pool2d(_t(x), k, s, p, d)
    np.testing.assert_array_equal(got.astype(np.float64), ref.numpy())


def test_maxpool_padding_is_minus_infinity():
    """All-negative input: zero padding would put 0 at the border, -inf padding does not."""
    x = -np.abs(inputgen.randn(5, (1, 1, 6, 6))) - 1.0
    y = oracle.maxpool2d(x, 4, 1, 1, 1)
    assert (y < -1.0).all()
    # an all-padding window gives -inf: H=W=1, k=2, d=2, p=1 -> taps at -1 and +1 only
    z = oracle.maxpool2d(np.ones((1, 1, 1, 1), np.float32), 2, 1, 1, 2)
    assert z.shape == (1, 1, 1, 1) and z[0, 0, 0, 0] == -np.inf


def test_maxpool_identity_and_separable():
    x = inputgen.randn(6, (2, 2, 9, 10))
    np.testing.assert_array_equal(oracle.maxpool2d(x, 1, 1, 0, 1), x)
    # l1_p42 page, the separable max: a row max followed by a column max equals
    # the 2-D max, bit for bit (max is exact)
    full = oracle.maxpool2d(x, 4, 1, 1, 1)
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)), constant_values=-np.inf)
    rowmax = np.maximum.reduce([xp[:, :, :, j: j + xp.shape[3] - 3] for j in range(4)])
    colmax = np.maximum.reduce([rowmax[:, :, i: i + rowmax.shape[2] - 3, :] for i in range(4)])
    np.testing.assert_array_equal(full, colmax)


def test_maxpool_result_is_in_window_and_dominates():
    x = inputgen.randn(8, (1, 2, 11, 11))
    k, s, p = 4, 1, 1
    y = oracle.maxpool2d(x, k, s, p, 1)
    xp = np.pad(x, ((0, 0), (0, 0), (p, p), (p, p)), constant_values=-np.inf)
    for c in range(2):
        for oh in range(y.shape[2]):
            for ow in range(y.shape[3]):
                win = xp[0, c, oh * s: oh * s + k, ow * s: ow * s + k]
                assert (y[0, c, oh, ow] >= win).all() and (win == y[0, c, oh, ow]).any()


# -------------------------------------------------------- fused conv + pool ---
def _torch_fused(c):
    y = F.conv2d(_t(c["x"]), _t(c["w"]), None if c["conv_bias"] is None else _t(c["conv_bias"]),
                 stride=c["conv_stride"], padding=c["conv_pad"], dilation=c["conv_dil"])
    y = torch.tanh(y)
    y = y * c["scale"]
    y = y + _t(c["bias2"]).view(1, -1, 1, 1)
    ps = c["pool_stride"] if c["pool_stride"] > 0 else c["pool_k"]
    return F.max_pool2d(y, c["pool_k"], ps, c["pool_pad"], c["pool_dil"]).numpy()


@pytest.mark.parametrize("kw", [
    dict(N=2, Cin=8, H=32, W=32, Cout=16),
    dict(N=1, Cin=3, H=19, W=23, Cout=5),
    dict(N=1, Cin=4, H=17, W=14, Cout=3, conv_pad=1, pool_k=3, pool_stride=2, pool_pad=1),
    dict(N=1, Cin=2, H=15, W=15, Cout=2, conv_stride=2, conv_dil=1, pool_k=2, pool_stride=2),
    dict(N=1, Cin=2, H=16, W=18, Cout=3, scale=-1.5),
    dict(N=1, Cin=2, H=12, W=12, Cout=3, conv_bias=False),
])
def test_fused_conv_pool_matches_torch_chain(kw):
    c = inputgen.random_conv_case(1000, **kw)
    got = oracle.conv_tanh_scale_bias_maxpool(c)
    np.testing.assert_allclose(got, _torch_fused(c), rtol=0, atol=1e-12)


def test_tiny_conv_workload_matches_torch_chain():
    c = inputgen.workload("tiny_conv")
    got = oracle.conv_tanh_scale_bias_maxpool(c)
    assert got.shape == (2, 16, 7, 7)
    np.testing.assert_allclose(got, _torch_fused(c), rtol=0, atol=1e-12)


def test_fused_points_equal_full():
    c = inputgen.random_conv_case(1100, N=2, Cin=3, H=21, W=18, Cout=4)
    full = oracle.conv_tanh_scale_bias_maxpool(c)
    idx = np.arange(full.size, dtype=np.int64)
    pts = oracle.conv_tanh_scale_bias_maxpool_points(c, idx)
    np.testing.assert_array_equal(pts, full.ravel())


@pytest.mark.parametrize("scale", [2.0, 0.5, -2.0, 0.0])
def test_monotone_reorder_identity(scale):
    """l2_p82 page, the argument that a nondecreasing pointwise map commutes with max:
    for scale > 0, max(tanh(y)*s + b) == tanh(max y)*s + b; for scale < 0 the max
    moves to the min of y; for scale == 0 the result is b.  Checked on the oracle's
    own conv values, so the oracle's written-order epilogue is pinned to the reordered
    form the GPU kernel uses."""
    c = inputgen.random_conv_case(1200, N=1, Cin=3, H=18, W=18, Cout=3, scale=scale)
    fused = oracle.conv_tanh_scale_bias_maxpool(c)
    y = oracle.conv2d(c["x"], c["w"], c["conv_bias"])
    win = y[:, :, :16, :16].reshape(1, 3, 4, 4, 4, 4)
    ymax = win.max(axis=(3, 5))
    ymin = win.min(axis=(3, 5))
    b2 = c["bias2"].astype(np.float64).reshape(1, -1, 1, 1)
    if scale > 0:
        alt = np.tanh(ymax) * scale + b2
    elif scale < 0:
        alt = np.tanh(ymin) * scale + b2
    else:
        alt = np.broadcast_to(b2, fused.shape)
    np.testing.assert_allclose(fused, alt, rtol=0, atol=1e-15)


# ---------------------------------------- second stage of the unfused conv ---
@pytest.mark.parametrize("k,st,p,d,scale", [(4, 4, 0, 1, 2.0), (3, 2, 1, 1, 2.0),
                                             (2, 1, 0, 2, -1.5), (3, 3, 1, 1, 0.0),
                                             (4, 1, 1, 1, 0.7)])
def test_tanh_scale_bias_maxpool_matches_torch_chain(k, st, p, d, scale):
    """The stored-conv-output epilogue + pool against torch fp64 (tanh, *scale, +bias,
    max_pool2d) on random data."""
    rng = np.random.default_rng(31)
    y = (rng.standard_normal((2, 3, 19, 17)) * 2).astype(np.float32)
    b2 = rng.standard_normal(3).astype(np.float32) * 0.1
    got = oracle.tanh_scale_bias_maxpool(y, b2, scale, k, st, p, d)
    z = torch.tanh(_t(y)) * scale + _t(b2).view(1, -1, 1, 1)
    ref = F.max_pool2d(z, k, st, p, d).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_two_stage_conv_equals_fused():
    """The l2_p82 page's unfused pipeline (conv to memory, then epilogue + pool)
    computes the fused op: oracle stage 2 on the oracle's conv output (rounded to
    float32, as a stored fp32 intermediate is) agrees with the fused oracle to the
    rounding of the intermediate."""
    c = inputgen.random_conv_case(1300, N=2, Cin=5, H=22, W=19, Cout=6, conv_pad=1,
                                  pool_k=3, pool_stride=2, pool_pad=1)
    y = oracle.conv2d(c["x"], c["w"], c["conv_bias"], c["conv_stride"], c["conv_pad"],
                      c["conv_dil"]).astype(np.float32)
    two = oracle.tanh_scale_bias_maxpool(y, c["bias2"], c["scale"], c["pool_k"],
                                         c["pool_stride"], c["pool_pad"], c["pool_dil"])
    np.testing.assert_allclose(two, oracle.conv_tanh_scale_bias_maxpool(c), rtol=0, atol=1e-6)


# ------------------------------------------------------- conv transpose 2d ---
@pytest.mark.parametrize("cfg", [
    dict(N=1, Cin=3, Cout=4, H=5, W=6, k=4, s=2, p=1, op=1, d=1),
    dict(N=2, Cin=2, Cout=3, H=4, W=4, k=4, s=2, p=1, op=0, d=1),
    dict(N=1, Cin=2, Cout=2, H=5, W=3, k=3, s=3, p=0, op=2, d=1),
    dict(N=1, Cin=2, Cout=2, H=4, W=5, k=3, s=2, p=2, op=1, d=2),
])
def test_conv_transpose_matches_torch_float64(cfg):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((cfg["N"], cfg["Cin"], cfg["H"], cfg["W"])).astype(np.float32)
    w = rng.uniform(-1, 1, (cfg["Cin"], cfg["Cout"], cfg["k"], cfg["k"])).astype(np.float32)
    b = rng.uniform(-1, 1, cfg["Cout"]).astype(np.float32)
    got = oracle.conv_transpose2d(x, w, b, cfg["s"], cfg["p"], cfg["op"], cfg["d"])
    ref = F.conv_transpose2d(_t(x), _t(w), _t(b), stride=cfg["s"], padding=cfg["p"],
                             output_padding=cfg["op"], dilation=cfg["d"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_conv_transpose_adjoint_identity():
    """<convT_w(x), g> == <x, conv_w(g)> with conv_w the k4 s2 p1 Conv2d of the same weight
    (w viewed as [out=Cin, in=Cout, k, k]); the l2_p91 page derives the transposed conv as the
    backward (gradient) of a forward conv."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 3, 6, 6)).astype(np.float32)
    w = rng.uniform(-1, 1, (3, 4, 4, 4)).astype(np.float32)
    y = oracle.conv_transpose2d(x, w, None, 2, 1, 1)
    assert y.shape == (1, 4, 13, 13)
    g = rng.standard_normal(y.shape).astype(np.float32)
    cg = oracle.conv2d(g, w, None, 2, 1, 1)
    assert cg.shape == x.shape
    lhs = float((y * g.astype(np.float64)).sum())
    rhs = float((x.astype(np.float64) * cg).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_conv_transpose_zero_insertion_form():
    """l2_p91 page, the zero-insertion view: insert s-1 zeros between input pixels, pad by
    d(k-1)-p (plus output_padding on the far side), then correlate with the kernel rotated
    by 180 degrees and with in/out channels swapped."""
    rng = np.random.default_rng(7)
    Cin, Cout, H, W, k, s, p, op = 2, 3, 5, 4, 4, 2, 1, 1
    x = rng.standard_normal((1, Cin, H, W)).astype(np.float32)
    w = rng.uniform(-1, 1, (Cin, Cout, k, k)).astype(np.float32)
    up = np.zeros((1, Cin, (H - 1) * s + 1, (W - 1) * s + 1), np.float64)
    up[:, :, ::s, ::s] = x
    e = k - 1 - p
    up = np.pad(up, ((0, 0), (0, 0), (e, e + op), (e, e + op)))
    wf = w[:, :, ::-1, ::-1].transpose(1, 0, 2, 3).astype(np.float64)  # [Cout, Cin, k, k]
    win = np.lib.stride_tricks.sliding_window_view(up, (k, k), axis=(2, 3))
    ref = np.einsum("nchwij,ocij->nohw", win, wf)
    got = oracle.conv_transpose2d(x, w, None, s, p, op)
    assert got.shape == ref.shape == (1, Cout, 2 * H + 1, 2 * W + 1)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def _golden_taps():
    rows, phases = {}, {}
    with open(os.path.join(GOLDEN, "convT_phase_taps.txt")) as f:
        for line in f:
            line = line.split("(")[0].strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("phase"):
                head, tail = line.split(":")
                _, a, b = head.split()
                phases[(int(a), int(b))] = {tuple(map(int, t.split(","))) for t in tail.split()}
            else:
                head, tail = line.split(":", 1)
                rows[int(head)] = {tuple(map(int, t.split(":"))) for t in tail.split()}
    return rows, phases


def test_conv_transpose_tap_table_from_page():
    """The oracle's index relation reproduces the page's printed row->tap table: a one-hot
    input row ih with a one-hot kernel row kh lands exactly on output row ih*2 - 1 + kh."""
    rows, phases = _golden_taps()
    H = 64
    found = {oh: set() for oh in rows}
    for kh in range(4):
        # one-hot kernel at (kh, kw=1): an input column iw=0 lands on output column 0
        w = np.zeros((1, 1, 4, 4), np.float32)
        w[0, 0, kh, 1] = 1.0
        x = np.zeros((1, 1, H, 1), np.float32)
        x[0, 0, :, 0] = np.arange(1, H + 1, dtype=np.float32)  # row id + 1
        y = oracle.conv_transpose2d(x, w, None, 2, 1, 1)[0, 0, :, 0]
        assert y.shape[0] == 129
        for oh in rows:
            if y[oh] != 0:
                found[oh].add((kh, int(y[oh]) - 1))
    assert found == rows
    # phase table: taps (kh, kw) touching output (oh, ow) of each parity
    for (a, b), taps in phases.items():
        got = set()
        for kh in range(4):
            for kw in range(4):
                w = np.zeros((1, 1, 4, 4), np.float32)
                w[0, 0, kh, kw] = 1.0
                y = oracle.conv_transpose2d(np.ones((1, 1, 8, 8), np.float32), w, None, 2, 1, 1)
                if y[0, 0, 2 + a, 2 + b] != 0:
                    got.add((kh, kw))
        assert got == taps


def test_conv_transpose_valid_pair_count():
    """k4 s2 p1 on 64 pixels: 64*4 (ih, kh) pairs per dimension minus the one landing at -1
    -> 255 valid pairs, so an all-ones input and kernel sum to 255^2."""
    y = oracle.conv_transpose2d(np.ones((1, 1, 64, 64), np.float32),
                                np.ones((1, 1, 4, 4), np.float32), None, 2, 1, 1)
    assert y.shape == (1, 1, 129, 129)
    assert y.sum() == 255 * 255


# --------------------------------------------- convT + softmax epilogue ---
def _torch_convT_chain(c):
    y = F.conv_transpose2d(_t(c["x"]), _t(c["w"]),
                           None if c["convT_bias"] is None else _t(c["convT_bias"]),
                           stride=c["stride"], padding=c["pad"],
                           output_padding=c["output_padding"], dilation=c["dil"])
    y = torch.softmax(y, dim=1)
    y = y + _t(c["bias2"]).view(1, -1, 1, 1)
    y = y * c["scale"]
    return torch.sigmoid(y).numpy()


@pytest.mark.parametrize("kw", [
    dict(N=2, Cin=4, H=5, W=6, Cout=8),
    dict(N=1, Cin=3, H=7, W=4, Cout=5, output_padding=0),
    dict(N=1, Cin=2, H=4, W=4, Cout=6, scale=-0.7, convT_bias=False),
])
def test_convT_softmax_chain_matches_torch(kw):
    c = inputgen.random_convT_case(2000, **kw)
    got = oracle.convT_softmax_bias_scale_sigmoid(c)
    np.testing.assert_allclose(got, _torch_convT_chain(c), rtol=0, atol=1e-13)


def test_softmax_sums_to_one_and_shift_invariance():
    c = inputgen.random_convT_case(2100, N=1, Cin=3, H=5, W=5, Cout=7)
    out = oracle.convT_softmax_bias_scale_sigmoid(c)
    s = c["scale"]
    sm = np.log(out / (1.0 - out)) / s - c["bias2"].astype(np.float64).reshape(1, -1, 1, 1)
    np.testing.assert_allclose(sm.sum(axis=1), 1.0, atol=1e-12)
    assert (sm > 0).all()
    c2 = dict(c)
    c2["convT_bias"] = (c["convT_bias"] + np.float32(3.0)).astype(np.float32)
    np.testing.assert_allclose(oracle.convT_softmax_bias_scale_sigmoid(c2), out, atol=1e-12)


def test_softmax_post_process_matches_torch_chain():
    """The stored-convT-output post-process against torch fp64 (softmax over dim 1,
    +bias, *scale, sigmoid)."""
    rng = np.random.default_rng(32)
    y = (rng.standard_normal((2, 9, 5, 7)) * 3).astype(np.float32)
    b2 = rng.standard_normal(9).astype(np.float32) * 0.1
    got = oracle.softmax_bias_scale_sigmoid(y, b2, -0.8)
    ref = torch.sigmoid((torch.softmax(_t(y), dim=1) + _t(b2).view(1, -1, 1, 1)) * -0.8)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-14)


def test_two_stage_convT_equals_fused():
    """The l2_p91 page's unfused pipeline (convT to memory, then the post-process)
    computes the fused op, up to the float32 rounding of the stored intermediate."""
    c = inputgen.random_convT_case(2300, N=2, Cin=4, H=5, W=6, Cout=8)
    y = oracle.conv_transpose2d(c["x"], c["w"], c["convT_bias"], c["stride"], c["pad"],
                                c["output_padding"], c["dil"]).astype(np.float32)
    two = oracle.softmax_bias_scale_sigmoid(y, c["bias2"], c["scale"])
    np.testing.assert_allclose(two, oracle.convT_softmax_bias_scale_sigmoid(c), rtol=0,
                               atol=1e-6)


def test_online_softmax_recurrence_equals_two_pass():
    """l2_p91 page, the one-pass running max / rescaled sum: when a larger value arrives,
    the running sum is multiplied by exp(old_max - new_max) before adding.  Pins the
    recurrence the GPU epilogue may use against the oracle's two-pass sum."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal(128) * 5
    m, s = -np.inf, 0.0
    for t in v:
        if t > m:
            s = s * math.exp(m - t) + 1.0 if m != -np.inf else 1.0
            m = t
        else:
            s += math.exp(t - m)
    assert m == v.max()
    assert abs(s - np.exp(v - v.max()).sum()) < 1e-12 * s


def test_convT_pixels_equal_full():
    c = inputgen.random_convT_case(2200, N=2, Cin=3, H=6, W=5, Cout=6)
    full = oracle.convT_softmax_bias_scale_sigmoid(c)
    N, C, OH, OW = full.shape
    pix = np.arange(N * OH * OW, dtype=np.int64)
    got = oracle.convT_softmax_bias_scale_sigmoid_pixels(c, pix)
    ref = full.transpose(0, 2, 3, 1).reshape(-1, C)
    np.testing.assert_allclose(got, ref, atol=1e-14)


# ------------------------------------------------------------- workloads ---
def test_workload_shapes():
    c = inputgen.workload("tiny_conv")
    assert oracle.conv_pool_out_shape(c) == (2, 16, 7, 7)
    small = dict(inputgen.random_conv_case(1, N=1, Cin=8, H=256, W=256, Cout=1))
    assert oracle.conv_pool_out_shape(small) == (1, 1, 63, 63)
    t = inputgen.random_convT_case(1, N=1, Cin=1, H=64, W=64, Cout=1)
    assert oracle.convT_out_shape(t) == (1, 1, 129, 129)


def test_bf16_rounding_is_rne():
    a = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1 + 1.5*2^-8 rounds up
    bits = inputgen.to_bf16_bits(a)
    back = inputgen.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0078125 and back[3] == 1.0078125
    assert back[4] == -2.5
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(back, ref)
