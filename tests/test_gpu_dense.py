"""GPU parity of the dense all-experts path (every token through every
expert, then the routed top-k combine) against the oracle's routed layer,
which the dense path must reproduce (KerasFormers "mxfp4" page, "As
GPT-OSS's native format": the routed and dense paths give identical output).

Bars as for the routed path: routing bit-exact outside rounding-level
near-ties; the output within 1e-2 * max|ref| (bf16 / fp32, fp32 also 1e-4)
and 3e-2 * max|ref| in the FP8 mode.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import compare_routing, device, note, oracle_full
from tests.test_gpu_layer import check_layer, fp8_20b_scales, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def test_dense_tiny_f32(dev):
    case = W.tiny()
    note(f"{case.name} dense")
    res, _, _ = run_gpu(case, dev, want_route=False, dense=True)
    check_layer(case, res, tol=1e-4)


@pytest.mark.parametrize("seed,E,H,I,k,T,act", [
    (40, 8, 64, 64, 2, 33, "bf16"),      # 264 rows over 8 experts: LDS-staged tiles, ragged last tile
    (41, 5, 96, 160, 3, 7, "bf16"),      # 35 rows: decode-shaped kernels with every expert active
    (42, 6, 160, 352, 2, 777, "bf16"),   # 4662 rows, 7 token tiles per expert
    (43, 3, 128, 96, 3, 5, "f32"),       # top_k = E: dense and routed run the same pairs
    (44, 16, 256, 128, 8, 40, "bf16"),   # top_k = 8
])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_dense_small_shapes(dev, seed, E, H, I, k, T, act, layout):
    case = W.small_case(seed, E, H, I, k, T, act_dtype=act)
    note(f"{case.name} {layout} dense")
    res, _, _ = run_gpu(case, dev, want_route=False, layout=layout, dense=True)
    check_layer(case, res, tol=1e-4 if act == "f32" else None)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_dense_decode_20b(dev, T):
    """The 20b shape (32 experts) at decode sizes: all 32 experts' weights
    are read for every token."""
    case = W.decode_20b(T=T)
    note(f"{case.name} tiled dense")
    res, _, _ = run_gpu(case, dev, want_route=False, layout="tiled", dense=True)
    check_layer(case, res)


def test_dense_fp8_20b(dev):
    """W-MXFP4 A-FP8 at T=2048 on the dense path (65536 GEMM rows); output of
    every token against the routed oracle (shared with the routed test)."""
    case = W.fp8_20b()
    s_x, s_h = fp8_20b_scales(case)
    note(f"{case.name} tiled dense")
    res, _, _ = run_gpu(case, dev, x_scale=s_x, h_scale=s_h, want_route=False, layout="tiled", dense=True)
    check_layer(case, res, x_scale=s_x, h_scale=s_h, full_ref=oracle_full(case, s_x, s_h))


def test_dense_matches_routed_on_gpu(dev):
    """Same routing bits on both paths, and outputs that differ only by the
    GEMMs' fp32 summation order (the kernels differ: per-expert token counts
    pick decode- or LDS-staged tiles)."""
    case = W.decode_20b(T=64)
    note(f"{case.name} tiled dense vs routed")
    rd, _, _ = run_gpu(case, dev, want_route=False, layout="tiled", dense=True)
    rr, _, _ = run_gpu(case, dev, want_route=False, layout="tiled", dense=False)
    assert np.array_equal(rd["idx"], rr["idx"]) and np.array_equal(rd["w"], rr["w"])
    compare_routing(case, rd["idx"], rd["w"])
    a = O.bf16_from_bits(rd["out"])
    b = O.bf16_from_bits(rr["out"])
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(b))


def test_dense_prefill_120b(dev):
    """The 120b prefill (T=4096, 128 experts) on the dense path: 524288 GEMM
    rows, whose h and Y (3 GB each) lie beyond one 32-bit buffer window, so
    the down GEMM's tiles address h through windows of their own rows.
    Every token against the routed oracle."""
    case = W.prefill_120b()
    note(f"{case.name} tiled dense")
    res, _, _ = run_gpu(case, dev, want_route=False, layout="tiled", dense=True)
    check_layer(case, res, full_ref=oracle_full(case))
