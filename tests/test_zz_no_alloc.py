"""GPU test of moe_mxfp4_forward_noalloc: through the C ABI, its output
matches moe_mxfp4_forward's (same kernels, so the same bits) on two calls in
a row, the second with a smaller batch, for the bf16 and FP8 modes."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_noalloc_matches_workspace_forward(dev, fp8, layout):
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.decode_20b(T=64)
    wts = W.layer_to_torch(case.layer, dev)
    if layout == "tiled":
        wts = wts.tiled()
    kw = {}
    if fp8:
        xc = W.fp8_20b().x_calib
        sc = W.torch_to_array(mx.moe_mxfp4_calibrate_fp8(wts, W.array_to_torch(xc, dev)))
        kw = dict(fp8=True, x_scale=float(sc[0]), h_scale=float(sc[1]))
    x = W.array_to_torch(case.x, dev)
    for T in (64, 5):  # the second call smaller than the first
        assert mx.workspace_bytes(wts, T, x.dtype, fp8) <= mx.NOALLOC_SCRATCH_BYTES
        note(f"noalloc {case.name} {layout} fp8={fp8} T={T}")
        xt = x[:T].contiguous()
        ref = mx.moe_mxfp4_forward(wts, xt, **kw)
        out = torch.empty_like(xt)
        idx = torch.empty((T, 4), dtype=torch.int32, device=dev)
        got = mx.moe_mxfp4_forward_noalloc(wts, xt, out, topk_idx_out=idx, **kw)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        assert np.all(np.isfinite(O.bf16_from_bits(W.torch_to_array(got))))
        assert W.torch_to_array(idx).min() >= 0


def test_noalloc_refuses_oversize_batch(dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.decode_20b(T=1)
    wts = W.layer_to_torch(case.layer, dev)
    x = torch.zeros((4096, 2880), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(x, 3.0)
    with pytest.raises(mx.MxmoeError) as ei:
        mx.moe_mxfp4_forward_noalloc(wts, x, out)
    assert ei.value.status == 5  # MXMOE_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
