"""The library's calls on several streams and inside HIP graphs.

The entry points keep no state and allocate nothing, so calls on different streams
are independent and a call can be captured into a graph.  Checked here:
  - the fused conv, the max-pool and the fused convT issued on two streams at once
    give the same bits as when issued one at a time;
  - the same three calls captured into one graph and replayed several times, with
    eager work and synchronisations between the replays, give the eager result on
    every replay (bit for bit: the kernels are deterministic).
Each case prints its name before its first GPU call.
"""
import sys

import numpy as np
import pytest

import inputgen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pool_stencil_amd  # noqa: F401
    return torch.device("cuda:0")


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _inputs(dev):
    import torch

    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    c = inputgen.random_conv_case(8000, N=4, Cin=8, H=66, W=130, Cout=64)
    t = inputgen.random_convT_case(8001, N=2, Cin=64, H=12, W=20, Cout=128)
    xp = put(inputgen.randn(8002, (4, 16, 70, 90)))
    return (dict(x=put(c["x"]), w=put(c["w"]), cb=put(c["conv_bias"]), b2=put(c["bias2"])),
            dict(x=put(t["x"]), w=put(t["w"]), cb=put(t["convT_bias"]), b2=put(t["bias2"])),
            xp)


def _run(ps, c, t, xp, outs, stream=None):
    ps.conv_tanh_scale_bias_maxpool(c["x"], c["w"], c["cb"], c["b2"], 2.0, 4, out=outs[0],
                                    stream=stream)
    ps.maxpool2d(xp, 4, 1, 1, 1, out=outs[1], stream=stream)
    ps.convT_softmax_bias_scale_sigmoid(t["x"], t["w"], t["cb"], t["b2"], 2.0, out=outs[2],
                                        stream=stream)


def _outs(dev):
    import torch
    return [torch.full((4, 64, 16, 32), float("nan"), device=dev),
            torch.full((4, 16, 69, 89), float("nan"), device=dev),
            torch.full((2, 128, 25, 41), float("nan"), device=dev)]


def test_two_streams(dev):
    import pool_stencil_amd as ps
    import torch
    _say("two streams")
    c, t, xp = _inputs(dev)
    ref = _outs(dev)
    _run(ps, c, t, xp, ref)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1, o2 = _outs(dev), _outs(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        _run(ps, c, t, xp, o1, stream=s1)
    with torch.cuda.stream(s2):
        _run(ps, c, t, xp, o2, stream=s2)
    torch.cuda.synchronize()
    for a, b, r in zip(o1, o2, ref):
        assert torch.equal(a, r) and torch.equal(b, r)


def test_graph_capture_and_replay(dev):
    import pool_stencil_amd as ps
    import torch
    _say("graph capture")
    c, t, xp = _inputs(dev)
    ref = _outs(dev)
    _run(ps, c, t, xp, ref)
    torch.cuda.synchronize()
    outs = _outs(dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        _run(ps, c, t, xp, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(ps, c, t, xp, outs)
    scratch = torch.empty(1 << 20, device=dev)
    for replay in range(3):
        for o in outs:
            o.fill_(float("nan"))
        scratch.normal_()                  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {replay}"
