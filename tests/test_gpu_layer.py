"""GPU parity of routing and of the whole MoE layer against the oracle.

Bars: routing index sets and the expert grouping are bit-exact (outside
rounding-level near-ties, reported); the layer output satisfies
max|d| <= 1e-2 * max|ref| for bf16/fp32 activations and <= 3e-2 * max|ref|
in the FP8-activation mode, ref being the oracle's unrounded float64
output.  The fp32 path is also held to 1e-4, the size of its own fp32
accumulation error over K <= 2880 (decoded weights and fp32 inputs are
exact, so only summation rounding remains).
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import compare_routing, device, max_rel_err, note, sub_case

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-2, "fp8": 3e-2}


@pytest.fixture(scope="module")
def dev():
    return device()


def run_gpu(case, dev, x_scale=1.0, h_scale=1.0, want_route=True, layout="rows", dense=False):
    import torch
    import mxfp4_quantized_moe_amd as mx

    wts = W.layer_to_torch(case.layer, dev)
    if layout == "tiled":
        wts = wts.tiled()
    x = W.array_to_torch(case.x, dev)
    T, k = case.T, case.layer.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = mx.moe_mxfp4_forward(wts, x, fp8=case.fp8, x_scale=x_scale, h_scale=h_scale, topk_idx_out=idx,
                               topk_w_out=w, dense=dense)
    torch.cuda.synchronize()
    res = dict(out=W.torch_to_array(out), idx=W.torch_to_array(idx), w=W.torch_to_array(w))
    if want_route:
        r = mx.moe_mxfp4_route(wts, x)
        torch.cuda.synchronize()
        res["route"] = [W.torch_to_array(t) for t in r]
    return res, wts, x


def as_f64(a, act):
    return O.bf16_from_bits(a) if act == "bf16" else a.astype(np.float64)


def boundary_tokens(case, route):
    """Tokens at the tile boundaries of the busiest expert (its first row,
    rows 127 and 128 of the sorted order: the last of its first 128-token
    tile and the first of the next, and its last row) and the first and last
    rows of the least busy expert with tokens."""
    idx, w, counts, offsets, sorted_slots, pos = route
    k = case.layer.top_k
    busy = [e for e in range(case.layer.E) if counts[e] > 0]
    emax = max(busy, key=lambda e: counts[e])
    emin = min(busy, key=lambda e: counts[e])
    picks = []
    for e, rows in ((emax, (0, 127, 128, counts[emax] - 1)), (emin, (0, counts[emin] - 1))):
        for r in rows:
            if 0 <= r < counts[e]:
                picks.append(int(sorted_slots[offsets[e] + r]) // k)
    return picks


def check_perm(case, route):
    idx, w, counts, offsets, sorted_slots, pos = route
    c, o, s, p = O.permute(idx, case.layer.E)
    assert np.array_equal(counts, c) and np.array_equal(offsets, o)
    assert np.array_equal(sorted_slots, s) and np.array_equal(pos, p)


def check_layer(case, res, sample=None, x_scale=None, h_scale=None, tol=None):
    k = case.layer.top_k
    n_exempt, override = compare_routing(case, res["idx"], res["w"])
    if sample is None:
        sample = np.arange(case.T)
    sc = sub_case(case, sample)
    ov = (override[0][sample], override[1][sample])
    ref = O.moe_forward(sc.layer, sc.x, case.act_dtype, fp8=case.fp8, x_scale=x_scale, h_scale=h_scale,
                        route_override=ov)
    got = as_f64(res["out"][sample], case.act_dtype)
    assert np.all(np.isfinite(as_f64(res["out"], case.act_dtype)))
    err = max_rel_err(got, ref)
    kind = "fp8" if case.fp8 else case.act_dtype
    bar = tol if tol is not None else TOL[kind]
    note(f"{case.name}: max|d|/max|ref| = {err:.3e} (bar {bar}), exempt tokens {n_exempt}")
    assert err <= bar
    return err


# ------------------------------------------------------------ the five workloads


def test_tiny_f32(dev):
    case = W.tiny()
    note(case.name)
    res, _, _ = run_gpu(case, dev)
    check_perm(case, res["route"])
    check_layer(case, res, tol=1e-4)


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_20b(dev, T, layout):
    case = W.decode_20b(T=T)
    note(f"{case.name} {layout}")
    res, _, _ = run_gpu(case, dev, layout=layout)
    check_perm(case, res["route"])
    check_layer(case, res)


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_prefill_120b_full_size(dev, layout):
    """T=4096 at the 120b shape: routing and grouping for every token, the
    layer output on 12 tokens spread over the batch plus the tokens at the
    busiest and least busy experts' tile boundaries (the oracle computes
    them one by one; tokens are independent)."""
    case = W.prefill_120b()
    note(f"{case.name} {layout}")
    res, _, _ = run_gpu(case, dev, layout=layout)
    check_perm(case, res["route"])
    counts = res["route"][2]
    assert counts.max() > 3 * counts.mean()  # the router bias skews expert load
    spread = np.linspace(0, case.T - 1, 12).astype(int)
    sample = np.unique(np.concatenate([spread, boundary_tokens(case, res["route"])]))
    check_layer(case, res, sample=sample)


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_fp8_20b_full_size(dev, layout):
    """W-MXFP4 A-FP8 at T=2048: static scales from the 256-token calibration
    batch (the oracle's values, fed to both sides), output on 12 tokens
    spread over the batch plus the tile-boundary tokens."""
    case = W.fp8_20b()
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    note(f"{case.name} {layout} s_x={s_x} s_h={s_h}")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, layout=layout)
    spread = np.linspace(0, case.T - 1, 12).astype(int)
    sample = np.unique(np.concatenate([spread, boundary_tokens(case, res["route"])]))
    check_layer(case, res, sample=sample, x_scale=s_x, h_scale=s_h)


def test_fp8_calibration_scales(dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.fp8_20b()
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    note("fp8 calibration")
    wts = W.layer_to_torch(case.layer, dev)
    sc = mx.moe_mxfp4_calibrate_fp8(wts, W.array_to_torch(case.x_calib, dev))
    torch.cuda.synchronize()
    g = W.torch_to_array(sc)
    assert np.float32(g[0]) == np.float32(s_x)  # amax of bf16 inputs is exact
    assert abs(g[1] - s_h) <= 1e-2 * s_h  # h differs by accumulation order only


# --------------------------------------------------------------- sweeps / edges


@pytest.mark.parametrize("seed,E,H,I,k,T,act", [
    (10, 8, 64, 64, 2, 33, "bf16"),      # ragged T, decode-shaped kernels
    (11, 5, 96, 160, 3, 7, "bf16"),      # K/32 = 3 and 5: partial 128-K chunks
    (12, 3, 128, 96, 3, 5, "f32"),       # top_k = E
    (13, 1, 64, 32, 1, 9, "bf16"),       # a single expert
    (14, 16, 256, 128, 8, 40, "bf16"),   # top_k = 8
    (15, 4, 64, 96, 2, 300, "bf16"),     # prefill kernels, R = 192 < one 512-row stripe
    (16, 6, 160, 352, 2, 777, "bf16"),   # prefill: ragged token tiles, K/32 = 5 and 11
    (17, 2, 32, 32, 1, 200, "bf16"),     # smallest dims through prefill
    (18, 4, 64, 64, 2, 130, "f32"),      # fp32 with more than 64 tokens per expert
    (19, 4, 96, 544, 2, 600, "bf16"),    # prefill: gate_up R = 1088 (2 stripes + a ragged third)
    (22, 100, 64, 64, 4, 20, "bf16"),    # router: 65 <= E <= 128 with few tokens (8 K-splitting waves)
    (23, 256, 64, 32, 8, 40, "bf16"),    # router: E = 256 (largest), top_k = 8
    (24, 200, 96, 64, 3, 70, "f32"),     # router: fp32 with E > 128
    (25, 8, 64, 32, 2, 3000, "bf16"),    # grouping: > 2048 slots (one workgroup per expert)
    (26, 256, 64, 32, 8, 600, "bf16"),   # grouping: > 2048 slots over 256 experts
    (37, 8, 64, 32, 2, 40000, "bf16"),   # grouping: > 65536 slots (expert ids re-read from global memory)
    (38, 8, 32, 32, 4, 270000, "bf16"),  # grouping: > 2^20 slots (back to the single-workgroup kernel)
    (27, 48, 160, 64, 4, 40, "f32"),     # router: fp32 with 32 < E <= 64 and few tokens (8 waves)
    (35, 4, 8192, 1024, 2, 300, "bf16"), # long K: 64 gate_up chunks through the prefill kernels
    (36, 4, 4096, 2048, 2, 5, "bf16"),   # long K through the decode kernels (32 and 16 chunks)
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_small_shapes(dev, seed, E, H, I, k, T, act, layout):
    case = W.small_case(seed, E, H, I, k, T, act_dtype=act)
    note(f"{case.name} {layout}")
    res, _, _ = run_gpu(case, dev, layout=layout)
    check_perm(case, res["route"])
    check_layer(case, res, tol=1e-4 if act == "f32" else None)


@pytest.mark.parametrize("seed,E,H,I,k,T", [
    (20, 4, 64, 64, 2, 16),     # decode-shaped
    (21, 4, 96, 160, 2, 400),   # prefill-shaped with partial chunks
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_small_fp8(dev, seed, E, H, I, k, T, layout):
    case = W.small_case(seed, E, H, I, k, T, act_dtype="bf16", fp8=True)
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    note(f"{case.name} fp8 {layout}")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, want_route=False, layout=layout)
    check_layer(case, res, x_scale=s_x, h_scale=s_h)


def test_empty_batch_is_noop(dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.small_case(30, 4, 64, 64, 2, 1)
    wts = W.layer_to_torch(case.layer, dev)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    out = mx.moe_mxfp4_forward(wts, x)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_deterministic_bits(dev):
    """Two forwards on the same inputs give identical bits (no float atomics)."""
    import torch
    import mxfp4_quantized_moe_amd as mx

    for case in (W.decode_20b(T=64), W.small_case(40, 8, 128, 96, 2, 500)):
        note(f"determinism {case.name}")
        wts = W.layer_to_torch(case.layer, dev)
        x = W.array_to_torch(case.x, dev)
        a = mx.moe_mxfp4_forward(wts, x).clone()
        b = mx.moe_mxfp4_forward(wts, x).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_prefixes_agree(dev):
    """T=1 and T=8 decode batches are prefixes of T=64; per-token results may
    only differ by the kernel path's rounding, not by routing."""
    import torch
    import mxfp4_quantized_moe_amd as mx

    c64 = W.decode_20b(T=64)
    wts = W.layer_to_torch(c64.layer, dev)
    x = W.array_to_torch(c64.x, dev)
    o64 = mx.moe_mxfp4_forward(wts, x)
    o8 = mx.moe_mxfp4_forward(wts, x[:8].contiguous())
    torch.cuda.synchronize()
    a = O.bf16_from_bits(W.torch_to_array(o64[:8]))
    b = O.bf16_from_bits(W.torch_to_array(o8))
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(a))


def test_skewed_routing_clamped_xcd_ranges(dev):
    """A router bias of std 3 sends almost every token to a few experts and
    leaves several with a handful: weighted by estimated work, one XCD's
    range of gate_up items would exceed the grid's workgroups per XCD, so
    the tiled kernel's clamp decides the split (checked on the oracle's
    routing with the host-side model of the split)."""
    from tests.test_xcd_split import TILE_COST, weighted_bounds

    case = W.small_case(33, 32, 128, 1024, 2, 2000, router_bias_std=3.0)
    L = case.layer
    idx, _, _ = O.route(O.bf16_from_bits(case.x), O.bf16_from_bits(L.router_w), O.bf16_from_bits(L.router_b), L.top_k)
    cnt = np.bincount(idx.reshape(-1), minlength=L.E).tolist()
    bnd, G, _, _, _ = weighted_bounds(cnt, 2 * L.I, TILE_COST)
    assert max(bnd[x + 1] - bnd[x] for x in range(8)) > G
    note(f"{case.name} tiled, expert counts {sorted(cnt)[-3:]} .. {sorted(cnt)[:3]}")
    res, _, _ = run_gpu(case, dev, layout="tiled")
    check_perm(case, res["route"])
    check_layer(case, res)


def test_fp8_saturating_activations(dev):
    """FP8 mode with x about 50x beyond the calibrated range: most codes of x
    saturate at +-448 on both sides (decided in fp32 from the same scale)."""
    case = W.small_case(34, 4, 96, 160, 2, 400, act_dtype="bf16", fp8=True)
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    case.x = O.bf16_bits(O.round_bf16(O.bf16_from_bits(case.x) * 50.0))
    assert np.mean(np.abs(O.bf16_from_bits(case.x)) / s_x > 448) > 0.5
    note(f"{case.name} fp8 saturating tiled")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, want_route=False, layout="tiled")
    check_layer(case, res, x_scale=s_x, h_scale=s_h)
