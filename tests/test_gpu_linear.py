"""GPU parity of the weight-only MXFP4 dense layer (mxfp4_linear) against
the oracle: max|d| <= 1e-2 * max|ref| with bf16 activations, <= 1e-4 with
fp32 ones (the fp32 accumulation error over K <= 2880), ref being the
oracle's unrounded float64 output."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import device, max_rel_err, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def run(case, dev, layout):
    import torch
    import mxfp4_quantized_moe_amd as mx

    N, K = case.blocks.shape[0], case.blocks.shape[1] * 32
    bias = W.array_to_torch(case.bias, dev) if case.bias is not None else None
    lin = mx.MXFP4Linear(W.array_to_torch(case.blocks, dev), W.array_to_torch(case.scales, dev), N, K, bias)
    if layout == "tiled":
        lin = lin.tiled()
    y = lin(W.array_to_torch(case.x, dev))
    torch.cuda.synchronize()
    return W.torch_to_array(y)


def as_f64(a, act):
    return O.bf16_from_bits(a) if act == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("seed,T,K,N,act,bias", [
    (1, 1, 64, 32, "bf16", True),       # one token: decode-shaped kernel
    (2, 7, 96, 64, "bf16", False),      # K/32 = 3: a partial 128-K chunk, no bias
    (3, 40, 2880, 544, "bf16", True),   # > 16 tokens: prefill tiles, N = 2 stripes + a ragged third
    (4, 300, 160, 96, "bf16", True),    # ragged token tiles (112, 96 and 92 rows)
    (5, 13, 128, 96, "f32", True),      # fp32 activations
    (6, 130, 64, 64, "f32", False),     # fp32, more than 64 tokens (token groups)
])
def test_linear_matches_oracle(dev, seed, T, K, N, act, bias, layout):
    case = W.linear_case(seed, T, K, N, act, bias)
    note(f"{case.name} {layout}")
    got = as_f64(run(case, dev, layout), act)
    ref = O.mxfp4_linear(case.x, case.blocks, case.scales, case.bias, act)
    assert np.all(np.isfinite(got))
    err = max_rel_err(got, ref)
    bar = 1e-4 if act == "f32" else 1e-2
    note(f"  max|d|/max|ref| = {err:.3e} (bar {bar})")
    assert err <= bar


def test_linear_full_size(dev):
    """The bench shape (T=4096, K=2880, N=5760, tiled): every output row."""
    case = W.linear_case(10, 4096, 2880, 5760, "bf16", True)
    note(case.name)
    got = as_f64(run(case, dev, "tiled"), "bf16")
    ref = O.mxfp4_linear(case.x, case.blocks, case.scales, case.bias, "bf16")
    assert np.all(np.isfinite(got))
    err = max_rel_err(got, ref)
    note(f"  max|d|/max|ref| = {err:.3e} over all rows (bar 1e-2)")
    assert err <= 1e-2
