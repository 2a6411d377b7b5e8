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
from tests.gpu_util import compare_routing, device, differing_sets, max_rel_err, note, oracle_full, poison, sub_case

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
    ws = mx.alloc_workspace(wts, T, x.dtype, case.fp8, dense)
    poison(ws)  # an intermediate row left unwritten turns the output NaN
    out = mx.moe_mxfp4_forward(wts, x, fp8=case.fp8, x_scale=x_scale, h_scale=h_scale, topk_idx_out=idx,
                               topk_w_out=w, dense=dense, workspace=ws)
    torch.cuda.synchronize()
    res = dict(out=W.torch_to_array(out), idx=W.torch_to_array(idx), w=W.torch_to_array(w))
    if want_route:
        r = mx.moe_mxfp4_route(wts, x)
        torch.cuda.synchronize()
        res["route"] = [W.torch_to_array(t) for t in r]
    return res, wts, x


def as_f64(a, act):
    return O.bf16_from_bits(a) if act == "bf16" else a.astype(np.float64)


def check_perm(case, route):
    idx, w, counts, offsets, sorted_slots, pos = route
    c, o, s, p = O.permute(idx, case.layer.E)
    assert np.array_equal(counts, c) and np.array_equal(offsets, o)
    assert np.array_equal(sorted_slots, s) and np.array_equal(pos, p)


def check_layer(case, res, x_scale=None, h_scale=None, tol=None, full_ref=None):
    """Every token of the GPU output against the oracle's.  full_ref: the
    oracle's (out, idx) over all tokens with its own routing (oracle_full);
    the few tokens where the GPU chose another expert set at a
    rounding-level near-tie are then recomputed with the GPU's choice.
    Without it the oracle runs over all tokens on the GPU's routing."""
    n_exempt, override = compare_routing(case, res["idx"], res["w"])
    kw = dict(fp8=case.fp8, x_scale=x_scale, h_scale=h_scale)
    if full_ref is None:
        ref = O.moe_forward(case.layer, case.x, case.act_dtype, route_override=override, **kw)
    else:
        ref = full_ref[0].copy()
        diff = differing_sets(res["idx"], full_ref[1])
        if diff.size:
            sc = sub_case(case, diff)
            ref[diff] = O.moe_forward(sc.layer, sc.x, case.act_dtype,
                                      route_override=(override[0][diff], override[1][diff]), **kw)
    got = as_f64(res["out"], case.act_dtype)
    assert np.all(np.isfinite(got))
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
    """T=4096 at the 120b shape: routing and grouping for every token and the
    layer output of every token (the oracle's float64 output over the whole
    batch, computed once for both layouts)."""
    case = W.prefill_120b()
    note(f"{case.name} {layout}")
    res, _, _ = run_gpu(case, dev, layout=layout)
    check_perm(case, res["route"])
    counts = res["route"][2]
    assert counts.max() > 3 * counts.mean()  # the router bias skews expert load
    check_layer(case, res, full_ref=oracle_full(case))


def fp8_20b_scales(case):
    key = ("calib", case.name)
    from tests import gpu_util as G

    if key not in G._REF_CACHE:
        G._REF_CACHE[key] = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    return G._REF_CACHE[key]


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_fp8_20b_full_size(dev, layout):
    """W-MXFP4 A-FP8 at T=2048: static scales from the 256-token calibration
    batch (the oracle's values, fed to both sides), output of every token."""
    case = W.fp8_20b()
    s_x, s_h = fp8_20b_scales(case)
    note(f"{case.name} {layout} s_x={s_x} s_h={s_h}")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, layout=layout)
    check_layer(case, res, x_scale=s_x, h_scale=s_h, full_ref=oracle_full(case, s_x, s_h))


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_fp8_by_hand(dev, layout):
    """The FP8 mode on the hand-derived layer of tests/hand_cases.py: the
    output must be exactly [0.875, 28, 0, ...] (router on the unquantised x,
    x and h quantised with their static scales, h saturating)."""
    from tests import hand_cases as HC

    case = HC.fp8_by_hand()
    note(f"{case.name} {layout}")
    res, _, _ = run_gpu(case, dev, x_scale=HC.FP8_X_SCALE, h_scale=HC.FP8_H_SCALE, want_route=False, layout=layout)
    assert res["idx"][0, 0] == 0 and res["w"][0, 0] == 1.0
    assert np.array_equal(O.bf16_from_bits(res["out"][0]), HC.FP8_EXPECTED)


def test_fp8_calibration_by_hand(dev):
    """GPU calibration on the hand-derived one-token batch: s_x has the bits
    of fp32(3/448) and s_h = 28/448 exactly."""
    import torch
    import mxfp4_quantized_moe_amd as mx
    from tests import hand_cases as HC

    case = HC.calib_by_hand()
    note(case.name)
    wts = W.layer_to_torch(case.layer, dev)
    sc = mx.moe_mxfp4_calibrate_fp8(wts, W.array_to_torch(case.x_calib, dev))
    torch.cuda.synchronize()
    g = W.torch_to_array(sc).astype(np.float32)
    assert g[0].view(np.uint32) == HC.CALIB_SX_BITS and g[1] == HC.CALIB_SH


def test_fp8_calibration_scales(dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.fp8_20b()
    s_x, s_h = fp8_20b_scales(case)
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
    (19, 4, 96, 544, 2, 600, "bf16"),    # prefill: gate_up R = 1088 (4 stripes + a ragged fifth of 64 rows)
    (29, 4, 128, 160, 2, 400, "bf16"),   # prefill: last stripes of 64 (gate_up) and 128 rows (down), full tiles
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
    (28, 4, 128, 160, 2, 400),  # last stripes of 64 and 128 rows with full token tiles
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_small_fp8(dev, seed, E, H, I, k, T, layout):
    case = W.small_case(seed, E, H, I, k, T, act_dtype="bf16", fp8=True)
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    note(f"{case.name} fp8 {layout}")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, want_route=False, layout=layout)
    check_layer(case, res, x_scale=s_x, h_scale=s_h)


@pytest.mark.parametrize("seed,T,act,fp8", [
    (71, 60, "bf16", False),   # experts with 21, 42 and 53 tokens
    (79, 60, "bf16", False),   # 15, 17, 21 and 55 tokens
    (86, 64, "bf16", False),   # one expert with 64 of the 128 slots (two full passes), others 16, 21
    (71, 60, "bf16", True),    # FP8 activations
    (71, 60, "f32", False),    # fp32 (row-order decode kernel only)
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_decode_kernels_many_tokens_per_expert(dev, seed, T, act, fp8, layout):
    """A strongly biased router at a decode-shaped batch (T*k <= 16 * min(E,
    T*k), so the decode-shaped kernels run) puts more than 32 tokens on one
    expert and 17..32 on another: the token passes past the first and the
    two-sub-tile passes of those kernels."""
    case = W.small_case(seed, 8, 128, 96, 2, T, act_dtype=act, fp8=fp8, router_bias_std=3.0)
    L = case.layer
    idx, _, _ = O.route(O.widen(case.x, act), O.widen(L.router_w, act), O.widen(L.router_b, act), L.top_k)
    cnt = np.bincount(idx.ravel(), minlength=L.E)
    assert T * L.top_k <= 16 * min(L.E, T * L.top_k)
    assert cnt.max() > 32 and np.any((cnt > 16) & (cnt <= 32))
    kw = {}
    if fp8:
        s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
        kw = dict(x_scale=s_x, h_scale=s_h)
    note(f"{case.name} {layout} {'fp8' if fp8 else act} counts {sorted(cnt.tolist())}")
    res, _, _ = run_gpu(case, dev, layout=layout, want_route=not fp8, **kw)
    if not fp8:
        check_perm(case, res["route"])
    check_layer(case, res, tol=1e-4 if act == "f32" else None, **kw)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_two_subtile_passes(dev, fp8):
    """A decode-shaped batch of more than 64 tokens (T=100, E=32, top-4)
    takes the decode tile with two 16-token sub-tiles per pass; a strongly
    biased router puts 100 tokens on some experts (four passes of 32) and
    17..32 on others (one two-sub-tile pass), and the combine is not folded
    (more than 64 tokens)."""
    T = 100
    case = W.small_case(103, 32, 128, 96, 4, T, act_dtype="bf16", fp8=fp8, router_bias_std=3.0)
    L = case.layer
    idx, _, _ = O.route(O.widen(case.x, "bf16"), O.widen(L.router_w, "bf16"), O.widen(L.router_b, "bf16"), L.top_k)
    cnt = np.bincount(idx.ravel(), minlength=L.E)
    assert T * L.top_k <= 16 * min(L.E, T * L.top_k)
    assert cnt.max() > 64 and np.any((cnt > 16) & (cnt <= 32))
    kw = {}
    if fp8:
        s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
        kw = dict(x_scale=s_x, h_scale=s_h)
    note(f"{case.name} tiled {'fp8' if fp8 else 'bf16'} counts {sorted(cnt.tolist())}")
    res, _, _ = run_gpu(case, dev, layout="tiled", want_route=not fp8, **kw)
    if not fp8:
        check_perm(case, res["route"])
    check_layer(case, res, **kw)


@pytest.mark.parametrize("seed, E, k, T, fp8, bias", [
    (122, 16, 8, 16, False, 0.01),   # 128 slots: positions ranked over two 64-slot rounds
    (126, 8, 8, 16, False, 3.0),     # every expert in every token: each expert's slots span both rounds
    (127, 64, 8, 16, False, 3.0),    # E = 64: all six id bits of the ballot ranking
    (124, 32, 4, 16, True, 0.01),    # FP8: the x codes written by the one router workgroup
    (120, 32, 4, 17, False, 0.01),   # one token past the one-workgroup batch: router + grouping launches
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_small_batch_grouping(dev, seed, E, k, T, fp8, bias, layout):
    """Batches of at most 16 tokens (E <= 64) are routed and grouped by the
    router's one workgroup: per-expert counts by LDS atomics and stable
    positions from ballots over the expert ids, 64 slots per round.
    Routing, grouping and the layer against the oracle, up to 128 slots and
    one token past that batch size."""
    case = W.small_case(seed, E, 128, 96, k, T, act_dtype="bf16", fp8=fp8, router_bias_std=bias)
    kw = {}
    if fp8:
        s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
        kw = dict(x_scale=s_x, h_scale=s_h)
    note(f"{case.name} {layout} {'fp8' if fp8 else 'bf16'}")
    res, _, _ = run_gpu(case, dev, layout=layout, want_route=not fp8, **kw)
    if not fp8:
        check_perm(case, res["route"])
    check_layer(case, res, **kw)


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


def test_workspace_reused_across_batches(dev):
    """One workspace through a sequence of forwards of different sizes, decode
    batches and one larger batch: every output equals that of a fresh
    workspace, bit for bit (nothing a forward leaves in its workspace may
    change the next one's result)."""
    import torch
    import mxfp4_quantized_moe_amd as mx

    c64 = W.decode_20b(T=64)
    wts = W.layer_to_torch(c64.layer, dev).tiled()
    x = W.array_to_torch(c64.x, dev)
    xl = W.array_to_torch(W.bf16_20b(300).x, dev)
    ws = mx.alloc_workspace(wts, 300, x.dtype)
    for T in (1, 64, 8, 300, 3, 64, 1):
        note(f"reused workspace T={T}")
        xt = (xl if T > 64 else x)[:T].contiguous()
        a = mx.moe_mxfp4_forward(wts, xt, workspace=ws)
        b = mx.moe_mxfp4_forward(wts, xt)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), T


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


# The library runs a tiled prefill GEMM as a persistent launch (512
# workgroups taking their XCD's item records through a counter) when the
# record grid holds at least 4 records per workgroup: max token tiles x row
# stripes of 256, rounded up to 8.
def record_blocks(case, R):
    rows = case.T * case.layer.top_k
    tiles = -(-rows // 128) + min(rows, case.layer.E)
    return -(-(tiles * -(-R // 256)) // 8) * 8


@pytest.mark.parametrize("seed,H,I,bias", [(41, 256, 2880, 0.01), (42, 2880, 256, 0.01), (43, 256, 2880, 1.5)])
def test_persistent_prefill_launches(dev, seed, H, I, bias):
    """T=4096, E=64, top-4 with one of the two GEMMs persistent: gate_up (2I
    = 5760 rows, 23 stripes) or down (H = 2880 rows, 12 stripes); the other
    runs one workgroup per record.  Every token against the oracle, on a
    poisoned workspace (an item no workgroup took leaves NaN rows).  Seed
    43 skews the routing so the XCDs' record lists differ in length."""
    case = W.small_case(seed, 64, H, I, 4, 4096, router_bias_std=bias)
    persistent = [record_blocks(case, R) >= 4 * 512 for R in (2 * I, H)]
    assert persistent == [I > H, H > I], persistent
    note(f"{case.name} tiled, persistent (gate_up, down) = {persistent}")
    res, _, _ = run_gpu(case, dev, layout="tiled")
    check_perm(case, res["route"])
    check_layer(case, res, full_ref=oracle_full(case))


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
