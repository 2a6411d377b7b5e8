"""GPU parity of the INT8 W8A8 MoE layer (int8 weights per output channel,
int8 activations per token, router and biases in bf16) against the
oracle, and of the 8-bit weight tiling against its test-side reference.

Bars: int8_tile bit-exact; routing bit-exact outside rounding-level
near-ties (as for the MXFP4 layer); the output within 1e-2 * max|ref|, ref
the oracle's unrounded float64 output on the GPU's routing.  x's int8 codes
are decided in fp32 on both sides from identical inputs; h's codes can
differ where the two sides' G straddles a rounding boundary, by one code.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import tiled_layout as TL
from tests.gpu_util import device, max_rel_err, note, poison

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def dev():
    return device()


def _run(case, dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    wts = W.int8_layer_to_torch(case.layer, dev)
    x = W.array_to_torch(case.x, dev)
    T, k = case.T, case.layer.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = torch.empty(max(mx.moe_int8_workspace_bytes(wts, T), 256), dtype=torch.uint8, device=dev)
    poison(ws)  # an intermediate row left unwritten turns the output NaN
    out = mx.moe_int8_forward(wts, x, topk_idx_out=idx, topk_w_out=w, workspace=ws)
    torch.cuda.synchronize()
    return W.torch_to_array(out), W.torch_to_array(idx), W.torch_to_array(w)


def _check_routing(case, gidx, gw, tau_rel=1e-4):
    """Set identity and weights where the k-th/(k+1)-th logit gap is above
    rounding level; else only experts within that gap.  Returns the GPU's
    choice with float64 softmax weights for the output check."""
    L = case.layer
    k = L.top_k
    xf = O.bf16_from_bits(case.x)
    idx, w, logits = O.route(xf, O.bf16_from_bits(L.router_w), O.bf16_from_bits(L.router_b), k)
    margin = O.routing_margin(logits, k)
    srt = -np.sort(-logits, axis=1)
    for t in range(case.T):
        tau = tau_rel * max(1.0, abs(srt[t, k - 1]))
        g = gidx[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < L.E
        if margin[t] >= tau:
            assert sorted(g.tolist()) == sorted(idx[t].tolist()), (t, g, idx[t])
            for j in range(k):
                jj = int(np.nonzero(idx[t] == g[j])[0][0])
                assert abs(gw[t, j] - w[t, jj]) <= 2e-6 * max(1.0, w[t, jj])
        else:
            assert np.all(logits[t, g] >= srt[t, k - 1] - tau)
    sel = np.take_along_axis(logits, gidx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return gidx.astype(np.int32), z / z.sum(axis=1, keepdims=True)


def _check(case, res):
    """Every token against the oracle on the GPU's routing."""
    out, gidx, gw = res
    ov = _check_routing(case, gidx, gw)
    ref = O.moe_forward_int8(case.layer, case.x, route_override=ov)
    got = O.bf16_from_bits(out)
    assert np.all(np.isfinite(got))
    err = max_rel_err(got, ref)
    note(f"{case.name}: max|d|/max|ref| = {err:.3e} (bar {TOL})")
    assert err <= TOL


@pytest.mark.parametrize("mats,rows,k", [(1, 32, 32), (2, 96, 160), (3, 64, 288)])
def test_int8_tile_bit_exact(dev, mats, rows, k):
    import torch
    import mxfp4_quantized_moe_amd as mx

    rng = np.random.default_rng(mats * 100 + rows + k)
    w = rng.integers(-127, 128, size=(mats, rows, k)).astype(np.int8)
    note(f"int8_tile {mats}x{rows}x{k}")
    t = mx.int8_tile(W.array_to_torch(w, dev))
    torch.cuda.synchronize()
    ref = np.concatenate([TL.fp8_tile(w[m].view(np.uint8)).reshape(-1) for m in range(mats)])
    assert np.array_equal(W.torch_to_array(t).reshape(-1), ref)


@pytest.mark.parametrize("seed,E,H,I,k,T", [
    (60, 8, 64, 64, 2, 33),       # ragged token tiles
    (61, 5, 96, 160, 3, 7),       # K/128 ragged, few tokens
    (62, 6, 160, 352, 2, 777),    # several token tiles per expert, K/32 = 5 and 11
    (63, 16, 256, 128, 8, 40),    # top_k = 8
    (64, 3, 128, 96, 3, 5),       # top_k = E
    (66, 4, 128, 160, 2, 400),    # last stripes of 64 (gate_up) and 128 rows (down), full token tiles
])
def test_int8_small_shapes(dev, seed, E, H, I, k, T):
    case = W.int8_case(seed, E, H, I, k, T)
    note(case.name)
    _check(case, _run(case, dev))


@pytest.mark.parametrize("T", [1, 8, 64])
def test_int8_20b_decode_sizes(dev, T):
    """Decode batches at the 20b shape: the decode-shaped int8 tile, with
    the combine folded into the down GEMM."""
    case = W.int8_20b(T)
    note(case.name)
    _check(case, _run(case, dev))


@pytest.mark.parametrize("seed,E,k,T", [
    (226, 8, 2, 60),    # one 16-token sub-tile per pass; experts with 32, 39 and 49 tokens
    (205, 32, 4, 100),  # two sub-tiles per pass (more than 64 tokens); 19 and 100 tokens
])
def test_int8_decode_many_tokens_per_expert(dev, seed, E, k, T):
    """Decode-shaped INT8 batches with a strongly biased router: experts past
    one token pass and with 17..32 tokens, on the int8 decode tile."""
    case = W.int8_case(seed, E, 128, 96, k, T, router_bias_std=3.0)
    L = case.layer
    idx, _, _ = O.route(O.bf16_from_bits(case.x), O.bf16_from_bits(L.router_w), O.bf16_from_bits(L.router_b), k)
    cnt = np.bincount(idx.ravel(), minlength=E)
    assert T * k <= 16 * min(E, T * k)
    assert cnt.max() > 32 and np.any((cnt > 16) & (cnt <= 32))
    note(f"{case.name} counts {sorted(cnt.tolist())}")
    _check(case, _run(case, dev))


def test_int8_20b_full_size(dev):
    """T=2048 at the 20b shape: routing and the output of every token."""
    case = W.int8_20b(2048)
    note(case.name)
    _check(case, _run(case, dev))


def test_int8_zero_token_rows(dev):
    """All-zero token rows quantise to scale 0 and codes 0 (no 0/0): their
    logits are the router bias alone and their gate_up output is the bias."""
    case = W.int8_case(65, 6, 128, 96, 2, 20)
    case.x[[0, 7, 19]] = 0
    note(case.name + " with zero rows 0, 7, 19")
    res = _run(case, dev)
    assert np.all(np.isfinite(O.bf16_from_bits(res[0])))
    _check(case, res)
