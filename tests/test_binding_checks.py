"""The Python binding checks tensor shapes, dtypes and devices before any
pointer reaches the library (CPU only: every check raises ValueError before
the device-pointer step, so host tensors suffice).

The C ABI takes sizes, not shapes, so a tensor smaller than its sizes say
would be read or written past its end by the kernels; these are the checks
that stop that in the binding.
"""
import pytest
import torch

import mxfp4_quantized_moe_amd as mx
from mxfp4_quantized_moe_amd import binding as B

E, H, I, K = 4, 64, 96, 2


def _layer(dtype=torch.bfloat16, **over):
    u8 = torch.uint8
    t = dict(
        gate_up_blocks=torch.zeros((E, 2 * I, H // 32, 16), dtype=u8),
        gate_up_scales=torch.zeros((E, 2 * I, H // 32), dtype=u8),
        gate_up_bias=torch.zeros((E, 2 * I), dtype=dtype),
        down_blocks=torch.zeros((E, H, I // 32, 16), dtype=u8),
        down_scales=torch.zeros((E, H, I // 32), dtype=u8),
        down_bias=torch.zeros((E, H), dtype=dtype),
        router_w=torch.zeros((E, H), dtype=dtype),
        router_b=torch.zeros((E,), dtype=dtype),
    )
    t.update(over)
    return mx.MoEWeights(**t, top_k=K)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_valid_layer_reaches_the_device_check():
    # a consistent layer passes every shape check and stops at the GPU check
    _raises(lambda: mx.moe_mxfp4_forward(_layer(), torch.zeros((3, H), dtype=torch.bfloat16)), "GPU tensors")


@pytest.mark.parametrize("field,bad", [
    ("gate_up_blocks", torch.zeros((E, 2 * I, H // 32 - 1, 16), dtype=torch.uint8)),
    ("gate_up_scales", torch.zeros((E, 2 * I, H // 32), dtype=torch.int8)),
    ("down_blocks", torch.zeros((E, H - 32, I // 32, 16), dtype=torch.uint8)),
    ("down_scales", torch.zeros((E, H, I // 32 + 1), dtype=torch.uint8)),
    ("down_bias", torch.zeros((E, H), dtype=torch.float32)),      # dtype differs from the router's
    ("router_b", torch.zeros((E + 1,), dtype=torch.bfloat16)),
])
def test_layer_tensor_mismatch(field, bad):
    layer = _layer(**{field: bad})
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=torch.bfloat16)), field)


def test_tiled_layer_too_small():
    layer = _layer()
    gb, gs = mx.mxfp4_tiled_bytes(E, 2 * I, H)
    db, ds = mx.mxfp4_tiled_bytes(E, H, I)
    u8 = torch.uint8
    tl = mx.MoEWeights(torch.zeros(gb, dtype=u8), torch.zeros(gs, dtype=u8), layer.gate_up_bias,
                       torch.zeros(db - 16, dtype=u8), torch.zeros(ds, dtype=u8), layer.down_bias,
                       layer.router_w, layer.router_b, top_k=K, layout=mx.LAYOUT_TILED)
    _raises(lambda: mx.moe_mxfp4_forward(tl, torch.zeros((3, H), dtype=torch.bfloat16)), "down_blocks")


def test_forward_x_and_out_shapes():
    layer = _layer()
    bf = torch.bfloat16
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H - 32), dtype=bf)), "x must be")
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=torch.float32)), "dtype")
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=bf), out=torch.zeros((2, H), dtype=bf)),
            "out must have shape")
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=bf), out=torch.zeros((3, H))),
            "out must be")
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=bf),
                                         topk_idx_out=torch.zeros((3, K), dtype=torch.int64)), "topk_idx_out")
    _raises(lambda: mx.moe_mxfp4_forward(layer, torch.zeros((3, H), dtype=bf),
                                         topk_w_out=torch.zeros((3, K + 1))), "topk_w_out")
    _raises(lambda: mx.moe_mxfp4_route(layer, torch.zeros((3, H + 32), dtype=bf)), "x must be")
    _raises(lambda: mx.moe_mxfp4_calibrate_fp8(_layer(torch.float32), torch.zeros((3, H))), "bf16")
    _raises(lambda: mx.ForwardPlan(layer, torch.zeros((3, H - 32), dtype=bf)), "x must be")


def test_linear_checks():
    N, Kd = 64, 96
    lin = mx.MXFP4Linear.from_rows(torch.zeros((N, Kd // 32, 16), dtype=torch.uint8),
                                   torch.zeros((N, Kd // 32), dtype=torch.uint8))
    _raises(lambda: mx.mxfp4_linear(torch.zeros((2, Kd - 32), dtype=torch.bfloat16), lin), "x must be")
    _raises(lambda: mx.mxfp4_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), lin,
                                    out=torch.zeros((2, N + 32), dtype=torch.bfloat16)), "out must have shape")
    bad_sc = mx.MXFP4Linear(lin.blocks, torch.zeros((N, Kd // 32 + 1), dtype=torch.uint8), N, Kd)
    _raises(lambda: mx.mxfp4_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), bad_sc), "scales")
    bad_b = mx.MXFP4Linear(lin.blocks, lin.scales, N, Kd, bias=torch.zeros((N,), dtype=torch.float32))
    _raises(lambda: mx.mxfp4_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), bad_b), "bias")
    _raises(lambda: mx.mxfp4_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), lin), "GPU tensors")


def test_fp8_linear_checks():
    N, Kd = 64, 128
    f = mx.FP8Linear(torch.zeros(mx.fp8_tiled_bytes(N, Kd) - 1, dtype=torch.uint8), N, Kd, 1.0, 1.0)
    _raises(lambda: mx.fp8_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), f), "w_tiled")
    f = mx.FP8Linear(torch.zeros(mx.fp8_tiled_bytes(N, Kd), dtype=torch.uint8), N, Kd, 1.0, 1.0)
    _raises(lambda: mx.fp8_linear(torch.zeros((2, Kd + 32), dtype=torch.bfloat16), f), "x must be")
    _raises(lambda: mx.fp8_linear(torch.zeros((2, Kd)), f), "x must be")
    _raises(lambda: mx.fp8_linear(torch.zeros((2, Kd), dtype=torch.bfloat16), f,
                                  out=torch.zeros((2, N), dtype=torch.float32)), "out must be")
    _raises(lambda: mx.fp8_tile(torch.zeros((N, Kd), dtype=torch.int8)), "w must be")


def test_int8_layer_checks():
    bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    n_gu, n_d = (B.ctypes.c_int64(0), B.ctypes.c_int64(0))
    lib = B.load_library()
    lib.int8_tiled_bytes(E, 2 * I, H, B.ctypes.byref(n_gu))
    lib.int8_tiled_bytes(E, H, I, B.ctypes.byref(n_d))
    good = dict(gate_up_w=torch.zeros(n_gu.value, dtype=u8), gate_up_scale=torch.zeros((E, 2 * I), dtype=f32),
                gate_up_bias=torch.zeros((E, 2 * I), dtype=bf), down_w=torch.zeros(n_d.value, dtype=u8),
                down_scale=torch.zeros((E, H), dtype=f32), down_bias=torch.zeros((E, H), dtype=bf),
                router_w=torch.zeros((E, H), dtype=bf), router_b=torch.zeros((E,), dtype=bf), top_k=K)
    x = torch.zeros((3, H), dtype=bf)
    _raises(lambda: mx.moe_int8_forward(mx.MoEInt8Weights(**good), x), "GPU tensors")
    for field, bad in (("down_scale", torch.zeros((E, H), dtype=bf)),
                       ("gate_up_w", torch.zeros(n_gu.value - 1, dtype=u8)),
                       ("router_b", torch.zeros((E - 1,), dtype=bf))):
        _raises(lambda: mx.moe_int8_forward(mx.MoEInt8Weights(**{**good, field: bad}), x), field)
    _raises(lambda: mx.moe_int8_forward(mx.MoEInt8Weights(**good), torch.zeros((3, H - 32), dtype=bf)), "x must be")
    _raises(lambda: mx.moe_int8_forward(mx.MoEInt8Weights(**good), x, out=torch.zeros((3, H))), "out must be")


def test_codec_checks():
    u8 = torch.uint8
    _raises(lambda: mx.mxfp4_unpack(torch.zeros((4, 3, 16), dtype=u8), torch.zeros((4, 2), dtype=u8)), "scales")
    _raises(lambda: mx.mxfp4_unpack(torch.zeros((4, 3, 8), dtype=u8), torch.zeros((4, 3), dtype=u8)), "blocks")
    _raises(lambda: mx.mxfp4_unpack(torch.zeros((4, 3, 16), dtype=u8), torch.zeros((4, 3), dtype=u8),
                                    out=torch.zeros((4, 64), dtype=torch.bfloat16)), "out must have shape")
    _raises(lambda: mx.mxfp4_pack(torch.zeros((4, 64), dtype=torch.float16)), "unsupported dtype")
    _raises(lambda: mx.mxfp4_tile(torch.zeros((2, 4, 3, 16), dtype=u8), torch.zeros((2, 4, 2), dtype=u8)), "scales")
