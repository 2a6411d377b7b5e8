"""The forward replayed from a HIP graph (the launch mode the benchmark times
for its layer workloads) against the same forward called directly.

Each graph is replayed several times with the program's own work between
the replays (the output cleared, the input changed, direct forwards on the
same workspace, synchronisations); every replay must equal the direct
result bit for bit, and the direct result is held to the oracle by the
layer tests.
"""
import pytest

import workloads as W
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _replays(case, dev, T, fp8_scales=None, layout="tiled", dense=False):
    import torch
    import mxfp4_quantized_moe_amd as mx

    wts = W.layer_to_torch(case.layer, dev)
    if layout == "tiled":
        wts = wts.tiled()
    xa = W.array_to_torch(case.x, dev)[:T].contiguous()
    xb = torch.flip(W.array_to_torch(case.x, dev)[-T:], dims=(0,)).contiguous()  # a second batch
    kw = dict(dense=dense)
    if fp8_scales is not None:
        kw.update(fp8=True, x_scale=fp8_scales[0], h_scale=fp8_scales[1])
    ref = {n: mx.moe_mxfp4_forward(wts, x, **kw) for n, x in (("a", xa), ("b", xb))}
    torch.cuda.synchronize()

    x = xa.clone()
    out = torch.empty_like(x)
    ws = mx.alloc_workspace(wts, T, x.dtype, fp8_scales is not None, dense)
    plan = mx.ForwardPlan(wts, x, out=out, workspace=ws, **kw)
    plan()  # a direct call ahead of the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        plan()
    for r, name in enumerate("abab"):
        note(f"{case.name} T={T} replay {r} input {name}")
        x.copy_(xa if name == "a" else xb)
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[name].view(torch.int16)), (r, name)
        # direct work on the same workspace between the replays
        direct = plan()
        torch.cuda.synchronize()
        assert torch.equal(direct.view(torch.int16), ref[name].view(torch.int16)), (r, name)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_graph_decode(dev, T):
    _replays(W.decode_20b(T=64), dev, T)


def test_graph_fp8(dev):
    case = W.fp8_20b()
    _replays(case, dev, 256, fp8_scales=(0.02, 0.05))


def test_graph_prefill_rows_layout(dev):
    _replays(W.bf16_20b(T=300), dev, 300, layout="rows")


def test_graph_persistent_prefill(dev):
    """A persistent gate_up launch (E=64, 2I = 5760 rows, T=4096): its list
    counters are set by the grouping kernel inside the graph, so every
    replay takes the same items."""
    _replays(W.small_case(44, 64, 256, 2880, 4, 4096), dev, 4096)


def test_graph_dense(dev):
    _replays(W.decode_20b(T=64), dev, 8, dense=True)
