"""GPU parity of the dense FP8 E4M3 layer (W8A8, static per-tensor scales)
against the oracle, and of the FP8 weight tiling against its test-side
reference.

Bars: fp8_tile bit-exact.  fp8_linear: max|d| <= 4e-3 * max|ref|, ref the
oracle's unrounded float64 output.  Both sides quantise x with the same
fp32 rule, so only the GEMM's fp32 summation order and the final bf16
rounding (half an ulp, 2^-9 relative) separate them.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import tiled_layout as TL
from tests.gpu_util import device, max_rel_err, note

pytestmark = pytest.mark.gpu

TOL = 4e-3


@pytest.fixture(scope="module")
def dev():
    return device()


def _run(case, dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    w = W.array_to_torch(case.w_codes, dev)
    b = W.array_to_torch(case.bias, dev) if case.bias is not None else None
    lin = mx.FP8Linear.from_codes(w, case.w_scale, case.x_scale, b)
    x = W.array_to_torch(case.x, dev)
    out = lin(x)
    torch.cuda.synchronize()
    return O.bf16_from_bits(W.torch_to_array(out))


@pytest.mark.parametrize("N,K", [(32, 32), (96, 160), (160, 288), (64, 2880)])
def test_fp8_tile_bit_exact(dev, N, K):
    import torch
    import mxfp4_quantized_moe_amd as mx

    rng = np.random.default_rng(N * 7 + K)
    w = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    note(f"fp8_tile N={N} K={K}")
    t = mx.fp8_tile(W.array_to_torch(w, dev))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_array(t).reshape(-1), TL.fp8_tile(w).reshape(-1))


@pytest.mark.parametrize("seed,T,K,N,bias", [
    (50, 1, 64, 64, True),        # one token
    (51, 5, 96, 64, False),       # K/128 ragged (partial last chunk), no bias
    (52, 200, 160, 96, True),     # two token tiles, N not a multiple of 64
    (53, 777, 288, 160, True),    # ragged token tiles, 3 chunks
    (54, 130, 2880, 512, True),   # the projection's contracting size
])
def test_fp8_linear_small(dev, seed, T, K, N, bias):
    case = W.fp8_linear_case(seed, T, K, N, bias=bias)
    note(case.name)
    got = _run(case, dev)
    ref = O.fp8_linear(case.x, case.w_codes, case.w_scale, case.x_scale, case.bias)
    err = max_rel_err(got, ref)
    note(f"{case.name}: max|d|/max|ref| = {err:.3e} (bar {TOL})")
    assert np.all(np.isfinite(got)) and err <= TOL


def test_fp8_linear_full_size(dev):
    """T=4096 through a 2880 -> 5760 projection, in the launch configuration
    the benchmark times; every output row."""
    case = W.fp8_linear_case(55, 4096, 2880, 5760)
    note(case.name)
    got = _run(case, dev)
    ref = O.fp8_linear(case.x, case.w_codes, case.w_scale, case.x_scale, case.bias)
    err = max_rel_err(got, ref)
    note(f"{case.name}: max|d|/max|ref| = {err:.3e} over all rows (bar {TOL})")
    assert np.all(np.isfinite(got)) and err <= TOL


def test_fp8_linear_saturates_inputs(dev):
    """Inputs far beyond 448 * x_scale saturate to +-448 on both sides."""
    case = W.fp8_linear_case(56, 40, 64, 64)
    x = O.bf16_from_bits(case.x) * 1000.0  # |x| up to ~4e3, 448 * 2^-6 = 7
    case.x = O.bf16_bits(O.round_bf16(x))
    note(case.name + " saturating")
    got = _run(case, dev)
    ref = O.fp8_linear(case.x, case.w_codes, case.w_scale, case.x_scale, case.bias)
    assert max_rel_err(got, ref) <= TOL
