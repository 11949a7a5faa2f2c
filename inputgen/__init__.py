"""Seeded synthetic inputs for the stencil workloads.

This module holds no arithmetic of the method itself: it only draws random
tensors (uniform, normal, Kaiming-uniform) from seeded numpy generators and
rounds fp32 data to bfloat16 where a workload stores bf16.  Both the oracle
tests and the HIP path take their inputs from here; nothing else is shared
between them.

Workloads (shapes and distributions follow the problem statements on the
three POPCORNBENCH pages; the suite's own problem files are not used):

  tiny_conv   x fp32 [2,8,32,32] U(-1,1); Conv2d 8->16 k3; w, conv bias
              U(+-1/sqrt(72)); bias2 [16] U(-0.1,0.1); scale 2; pool k4 s4
  maxpool     x fp32 [32,64,512,512] randn; MaxPool2d k4 s1 p1 d1
  conv        x fp32 [128,8,256,256] U(-1,1); Conv2d 8->64 k3; Kaiming-uniform
              w and conv bias (fan_in 72); bias2 randn*0.02; scale 2; pool k4 s4
  convT       x fp32 [128,64,64,64] randn; ConvTranspose2d 64->128 k4 s2 p1 op1;
              Kaiming-uniform w [64,128,4,4] and bias (fan_in 2048);
              bias2 randn*0.02; scale 2
  conv_bf16   as conv, with x and w rounded to bf16 (round-to-nearest-even)

Kaiming-uniform here means U(-1/sqrt(fan_in), +1/sqrt(fan_in)), PyTorch's
default initialisation for Conv2d / ConvTranspose2d parameters (not stated on
the pages; the problem statements only build the modules with defaults).
"""
from __future__ import annotations

import concurrent.futures as _cf
import math

import numpy as np

SEED_BASE = 0x5EED0000
_CHUNK = 1 << 22  # elements per independently seeded chunk (fixed: part of the stream definition)


def seed_for(workload_index: int, slot: int) -> int:
    """Seed of tensor `slot` (0 x, 1 w, 2 conv bias, 3 bias2) of workload `workload_index`."""
    return SEED_BASE + 16 * workload_index + slot


def _fill(seed: int, n: int, draw) -> np.ndarray:
    """Fill n float32 values chunk by chunk; chunk i uses child i of SeedSequence(seed)."""
    out = np.empty(n, dtype=np.float32)
    nchunk = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = np.random.SeedSequence(seed).spawn(nchunk)

    def work(i):
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        draw(np.random.Generator(np.random.PCG64(children[i])), out[lo:hi])

    if nchunk == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(max_workers=min(16, nchunk)) as ex:
            list(ex.map(work, range(nchunk)))
    return out


def uniform(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    """float32 U(lo, hi) of the given shape."""
    n = int(np.prod(shape)) if len(shape) else 1

    def draw(g, dst):
        g.random(out=dst, dtype=np.float32)
        dst *= np.float32(hi - lo)
        dst += np.float32(lo)

    return _fill(seed, n, draw).reshape(shape)


def randn(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) of the given shape."""
    n = int(np.prod(shape)) if len(shape) else 1

    def draw(g, dst):
        g.standard_normal(out=dst, dtype=np.float32)
        if std != 1.0:
            dst *= np.float32(std)

    return _fill(seed, n, draw).reshape(shape)


def kaiming_uniform(seed: int, shape, fan_in: int) -> np.ndarray:
    b = 1.0 / math.sqrt(fan_in)
    return uniform(seed, shape, -b, b)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, round-to-nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Workload table.  Index = position in the list of the five workloads.
# ---------------------------------------------------------------------------
WORKLOADS = ["tiny_conv", "maxpool", "conv", "convT", "conv_bf16", "conv_general", "convT_bf16"]


def _conv_case(idx, N, Cin, H, W, Cout, wdist, b2dist, dtype="f32", N_take=None):
    fan_in = Cin * 9
    x = uniform(seed_for(idx, 0), (N, Cin, H, W), -1.0, 1.0)
    w = kaiming_uniform(seed_for(idx, 1), (Cout, Cin, 3, 3), fan_in)
    cb = kaiming_uniform(seed_for(idx, 2), (Cout,), fan_in)
    if b2dist == "u0.1":
        b2 = uniform(seed_for(idx, 3), (Cout,), -0.1, 0.1)
    else:
        b2 = randn(seed_for(idx, 3), (Cout,), 0.02)
    case = dict(op="conv_pool", dtype=dtype, x=x, w=w, conv_bias=cb, bias2=b2,
                N=N, Cin=Cin, H=H, W=W, Cout=Cout, kH=3, kW=3,
                conv_stride=1, conv_pad=0, conv_dil=1, scale=2.0,
                pool_k=4, pool_stride=4, pool_pad=0, pool_dil=1)
    if dtype == "bf16":
        case["x_bits"] = to_bf16_bits(x)
        case["w_bits"] = to_bf16_bits(w)
        case["x"] = bf16_bits_to_f32(case["x_bits"]).reshape(x.shape)
        case["w"] = bf16_bits_to_f32(case["w_bits"]).reshape(w.shape)
    return case


def workload(name: str) -> dict:
    """Host arrays and parameters of one named workload (full size)."""
    idx = WORKLOADS.index(name)
    if name == "tiny_conv":
        x = uniform(seed_for(idx, 0), (2, 8, 32, 32), -1.0, 1.0)
        b = 1.0 / math.sqrt(72)
        w = uniform(seed_for(idx, 1), (16, 8, 3, 3), -b, b)
        cb = uniform(seed_for(idx, 2), (16,), -b, b)
        b2 = uniform(seed_for(idx, 3), (16,), -0.1, 0.1)
        return dict(op="conv_pool", dtype="f32", x=x, w=w, conv_bias=cb, bias2=b2,
                    N=2, Cin=8, H=32, W=32, Cout=16, kH=3, kW=3,
                    conv_stride=1, conv_pad=0, conv_dil=1, scale=2.0,
                    pool_k=4, pool_stride=4, pool_pad=0, pool_dil=1)
    if name == "maxpool":
        x = randn(seed_for(idx, 0), (32, 64, 512, 512))
        return dict(op="maxpool", dtype="f32", x=x, N=32, C=64, H=512, W=512,
                    k=4, stride=1, pad=1, dil=1)
    if name == "conv":
        return _conv_case(idx, 128, 8, 256, 256, 64, "kaiming", "randn0.02")
    if name == "conv_bf16":
        return _conv_case(idx, 128, 8, 256, 256, 64, "kaiming", "randn0.02", dtype="bf16")
    if name == "convT_bf16":
        # the convT workload's shapes and distributions, x and w rounded to bf16
        c = workload("convT")
        return _bf16_convT(dict(c))
    if name == "convT":
        fan_in = 128 * 16
        x = randn(seed_for(idx, 0), (128, 64, 64, 64))
        w = kaiming_uniform(seed_for(idx, 1), (64, 128, 4, 4), fan_in)
        cb = kaiming_uniform(seed_for(idx, 2), (128,), fan_in)
        b2 = randn(seed_for(idx, 3), (128,), 0.02)
        return dict(op="convT", dtype="f32", x=x, w=w, convT_bias=cb, bias2=b2,
                    N=128, Cin=64, H=64, W=64, Cout=128, k=4, stride=2, pad=1,
                    output_padding=1, dil=1, scale=2.0)
    if name == "conv_general":
        # The fused op beyond the 3x3 / 8-channel / disjoint-window case: 64 -> 128
        # channels, 3x3 conv with padding 1, overlapping 3x3 stride-2 pool with
        # padding 1; value distributions as in the conv workload.
        c = random_conv_case(seed_for(idx, 0), 32, 64, 128, 128, 128, conv_pad=1,
                             pool_k=3, pool_stride=2, pool_pad=1)
        return c
    raise KeyError(name)


def random_conv_case(seed: int, N, Cin, H, W, Cout, kH=3, kW=3, conv_stride=1, conv_pad=0,
                     conv_dil=1, scale=2.0, pool_k=4, pool_stride=4, pool_pad=0, pool_dil=1,
                     dtype="f32", conv_bias=True):
    """A small fused-conv case with the same value distributions as the conv workload."""
    fan_in = Cin * kH * kW
    x = uniform(seed, (N, Cin, H, W), -1.0, 1.0)
    w = kaiming_uniform(seed + 1, (Cout, Cin, kH, kW), fan_in)
    cb = kaiming_uniform(seed + 2, (Cout,), fan_in) if conv_bias else None
    b2 = randn(seed + 3, (Cout,), 0.02)
    case = dict(op="conv_pool", dtype=dtype, x=x, w=w, conv_bias=cb, bias2=b2,
                N=N, Cin=Cin, H=H, W=W, Cout=Cout, kH=kH, kW=kW,
                conv_stride=conv_stride, conv_pad=conv_pad, conv_dil=conv_dil, scale=scale,
                pool_k=pool_k, pool_stride=pool_stride, pool_pad=pool_pad, pool_dil=pool_dil)
    if dtype == "bf16":
        case["x_bits"] = to_bf16_bits(x)
        case["w_bits"] = to_bf16_bits(w)
        case["x"] = bf16_bits_to_f32(case["x_bits"]).reshape(x.shape)
        case["w"] = bf16_bits_to_f32(case["w_bits"]).reshape(w.shape)
    return case


def _bf16_convT(case):
    case["dtype"] = "bf16"
    case["x_bits"] = to_bf16_bits(case["x"])
    case["w_bits"] = to_bf16_bits(case["w"])
    case["x"] = bf16_bits_to_f32(case["x_bits"]).reshape(case["x"].shape)
    case["w"] = bf16_bits_to_f32(case["w_bits"]).reshape(case["w"].shape)
    return case


def random_convT_case(seed: int, N, Cin, H, W, Cout, k=4, stride=2, pad=1, output_padding=1,
                      dil=1, scale=2.0, convT_bias=True, dtype="f32"):
    fan_in = Cout * k * k
    x = randn(seed, (N, Cin, H, W))
    w = kaiming_uniform(seed + 1, (Cin, Cout, k, k), fan_in)
    cb = kaiming_uniform(seed + 2, (Cout,), fan_in) if convT_bias else None
    b2 = randn(seed + 3, (Cout,), 0.02)
    case = dict(op="convT", dtype="f32", x=x, w=w, convT_bias=cb, bias2=b2,
                N=N, Cin=Cin, H=H, W=W, Cout=Cout, k=k, stride=stride, pad=pad,
                output_padding=output_padding, dil=dil, scale=scale)
    return _bf16_convT(case) if dtype == "bf16" else case
