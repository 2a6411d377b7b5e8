"""The C ABI without a GPU: the library loads, exports what include/mxmoe.h
declares, and rejects bad arguments on the host before any launch.

Every call here fails validation (or is a documented no-op) so nothing is
launched; fake device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import mxfp4_quantized_moe_amd as mx
from mxfp4_quantized_moe_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")

OK, NULL, ALIGN, SHAPE, DTYPE, WS, UNSUP, HIP, VALUE = range(9)
P = 0x10000  # a 16-byte aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmxmoe.so is not built: run `python -m mxfp4_quantized_moe_amd.build`")
    return mx.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mxmoe_version() == 4
    for s in range(9):
        assert lib.mxmoe_status_string(s)


def test_unpack_pack_validation(lib):
    s = None
    assert lib.mxfp4_unpack(P, P, 4, 48, P, 1, s) == SHAPE  # k % 32 != 0 ("a clear error")
    assert lib.mxfp4_unpack(P, P, 4, 0, P, 1, s) == SHAPE
    assert lib.mxfp4_unpack(P, P, -1, 64, P, 1, s) == SHAPE
    assert lib.mxfp4_unpack(P, P, 4, 64, P, 7, s) == DTYPE
    assert lib.mxfp4_unpack(None, P, 4, 64, P, 1, s) == NULL
    assert lib.mxfp4_unpack(P, P, 4, 64, P + 8, 1, s) == ALIGN
    assert lib.mxfp4_unpack(P, P, 0, 64, P, 1, s) == OK  # no rows: no-op, nothing launched
    assert lib.mxfp4_pack(P, 0, 4, 33, P, P, s) == SHAPE
    assert lib.mxfp4_pack(P, 2, 4, 64, P, P, s) == DTYPE
    assert lib.mxfp4_pack(P, 0, 4, 64, None, P, s) == NULL
    assert lib.mxfp4_pack(P + 4, 0, 4, 64, P, P, s) == ALIGN
    assert lib.mxfp4_pack(P, 1, 0, 64, P, P, s) == OK


def test_tiled_bytes(lib):
    bb, sb = ctypes.c_int64(-1), ctypes.c_int64(-1)
    # gpt-oss gate_up: rows 5760 = 90 groups of 64, k 2880 = 90 blocks -> 23 chunks of 4 blocks
    assert lib.mxfp4_tiled_bytes(2, 5760, 2880, ctypes.byref(bb), ctypes.byref(sb)) == OK
    assert (bb.value, sb.value) == (2 * 360 * 23 * 1024, 2 * 90 * 23 * 256)
    # ragged: 70 rows -> 2 groups (8 row tiles), k 96 -> 3 blocks -> 1 chunk
    assert lib.mxfp4_tiled_bytes(3, 70, 96, ctypes.byref(bb), ctypes.byref(sb)) == OK
    assert (bb.value, sb.value) == (3 * 8 * 1 * 1024, 3 * 2 * 1 * 256)
    assert lib.mxfp4_tiled_bytes(0, 70, 96, ctypes.byref(bb), ctypes.byref(sb)) == OK and bb.value == 0
    assert lib.mxfp4_tiled_bytes(1, 64, 48, ctypes.byref(bb), ctypes.byref(sb)) == SHAPE
    assert lib.mxfp4_tiled_bytes(-1, 64, 64, ctypes.byref(bb), ctypes.byref(sb)) == SHAPE
    assert lib.mxfp4_tiled_bytes(1, 64, 64, None, ctypes.byref(sb)) == NULL


def test_tile_validation(lib):
    s = None
    assert lib.mxfp4_tile(P, P, 2, 64, 48, P, P, s) == SHAPE
    assert lib.mxfp4_tile(P, P, 2, -3, 64, P, P, s) == SHAPE
    assert lib.mxfp4_tile(None, P, 2, 64, 64, P, P, s) == NULL
    assert lib.mxfp4_tile(P, P, 2, 64, 64, P, None, s) == NULL
    assert lib.mxfp4_tile(P, P + 8, 2, 64, 64, P, P, s) == ALIGN
    assert lib.mxfp4_tile(P, P, 0, 64, 64, None, None, s) == OK  # nothing to tile: no-op
    assert lib.mxfp4_tile(P, P, 2, 0, 64, None, None, s) == OK


def _layer(**kw):
    d = dict(E=4, H=64, I=64, top_k=2, param_dtype=1, weight_layout=0, gate_up_blocks=P, gate_up_scales=P,
             gate_up_bias=P, down_blocks=P, down_scales=P, down_bias=P, router_w=P, router_b=P)
    d.update(kw)
    return B.Layer(**d)


def _opts(**kw):
    d = dict(act_dtype=1, fp8_act=0, x_scale=1.0, h_scale=1.0, topk_idx_out=None, topk_w_out=None)
    d.update(kw)
    return B.FwdOpts(**d)


def _fwd(lib, layer, T=8, opts=None, x=P, out=P, ws=P, ws_bytes=1 << 30):
    opts = opts or _opts()
    return lib.moe_mxfp4_forward(ctypes.byref(layer), x, T, out, ctypes.byref(opts), ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=48), SHAPE),            # contracting dim of gate_up not a multiple of 32
    (dict(I=80), SHAPE),            # contracting dim of down not a multiple of 32
    (dict(E=0), SHAPE),
    (dict(E=257), SHAPE),
    (dict(top_k=0), SHAPE),
    (dict(top_k=5), SHAPE),         # > E
    (dict(E=16, top_k=9), SHAPE),   # > 8
    (dict(param_dtype=3), DTYPE),
    (dict(weight_layout=2), VALUE),
    (dict(gate_up_blocks=None), NULL),
    (dict(router_b=None), NULL),
    (dict(down_scales=P + 1), ALIGN),
])
def test_forward_layer_validation(lib, kw, code):
    assert _fwd(lib, _layer(**kw)) == code


def test_forward_opts_validation(lib):
    L = _layer()
    assert _fwd(lib, L, opts=_opts(act_dtype=5)) == DTYPE
    assert _fwd(lib, L, opts=_opts(act_dtype=0)) == DTYPE  # x fp32 with bf16 params
    assert _fwd(lib, _layer(param_dtype=0), opts=_opts(act_dtype=0, fp8_act=1)) == DTYPE  # FP8 needs bf16
    assert _fwd(lib, L, opts=_opts(fp8_act=1, x_scale=0.0)) == VALUE
    assert _fwd(lib, L, opts=_opts(fp8_act=1, h_scale=float("nan"))) == VALUE
    assert _fwd(lib, L, opts=_opts(fp8_act=1, x_scale=-1.0)) == VALUE
    assert _fwd(lib, L, opts=_opts(fp8_act=2)) == VALUE
    assert _fwd(lib, L, opts=_opts(topk_idx_out=P + 4)) == ALIGN
    assert lib.moe_mxfp4_forward(ctypes.byref(L), P, 8, P, None, P, 1 << 30, None) == NULL


def test_forward_token_and_workspace_validation(lib):
    L = _layer()
    assert _fwd(lib, L, T=-1) == SHAPE
    assert _fwd(lib, L, T=0, x=None, out=None, ws=None) == OK  # empty batch: no-op
    assert _fwd(lib, L, x=None) == NULL
    assert _fwd(lib, L, out=P + 2) == ALIGN
    need = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 8, ctypes.byref(_opts()))
    assert need > 0
    assert _fwd(lib, L, ws_bytes=need - 1) == WS
    assert _fwd(lib, L, T=(1 << 26)) == SHAPE  # T * top_k beyond the slot limit
    # the FP8 mode needs room for the quantised x
    need8 = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 8, ctypes.byref(_opts(fp8_act=1)))
    assert need8 > need - 8 * 64 * 2 * 1
    assert lib.moe_mxfp4_workspace_bytes(ctypes.byref(_layer(H=40)), 8, ctypes.byref(_opts())) == 0


def test_forward_noalloc_validation(lib):
    """The no-allocation forward validates like moe_mxfp4_forward and refuses
    a batch whose workspace exceeds its fixed scratch array, before any
    launch and before it looks up the array's device address."""
    L = _layer()

    def fwd(layer=L, T=8, opts=None, x=P, out=P):
        opts = opts or _opts()
        return lib.moe_mxfp4_forward_noalloc(ctypes.byref(layer), x, T, out, ctypes.byref(opts), None)

    assert fwd(_layer(H=48)) == SHAPE
    assert fwd(_layer(router_b=None)) == NULL
    assert fwd(opts=_opts(act_dtype=0)) == DTYPE
    assert fwd(opts=_opts(fp8_act=1, x_scale=0.0)) == VALUE
    assert fwd(T=-1) == SHAPE
    assert fwd(T=0, x=None, out=None) == OK  # empty batch: no-op
    big = _layer(E=32, H=2880, I=2880, top_k=4)
    n = lib.moe_mxfp4_workspace_bytes(ctypes.byref(big), 4096, ctypes.byref(_opts()))
    assert n > B.NOALLOC_SCRATCH_BYTES
    assert fwd(big, T=4096) == WS
    # the header's figure and the binding's agree
    text = open(HEADER).read()
    assert re.search(r"#define MXMOE_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)
    assert B.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_dense_path_validation(lib):
    L = _layer(E=32, H=2880, I=2880, top_k=4)
    assert _fwd(lib, _layer(), opts=_opts(expert_path=2)) == VALUE
    assert _fwd(lib, _layer(), opts=_opts(expert_path=-1)) == VALUE
    routed = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 64, ctypes.byref(_opts()))
    dense = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 64, ctypes.byref(_opts(expert_path=1)))
    # h and Y for all T*E (expert, token) rows instead of T*k
    assert dense >= routed + 64 * (32 - 4) * (2880 * 2 + 2880 * 2)
    assert lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 64, ctypes.byref(_opts(expert_path=3))) == 0
    # the 120b prefill: T*E = 524288 rows of h and Y (3 GB each in bf16) are
    # more than one 32-bit buffer window reaches, but the kernels address h
    # one tile's rows at a time, so the dense path takes it
    big = _layer(E=128, H=2880, I=2880, top_k=4)
    routed_big = lib.moe_mxfp4_workspace_bytes(ctypes.byref(big), 4096, ctypes.byref(_opts()))
    dense_big = lib.moe_mxfp4_workspace_bytes(ctypes.byref(big), 4096, ctypes.byref(_opts(expert_path=1)))
    assert routed_big > 0
    assert dense_big >= routed_big + 4096 * (128 - 4) * (2880 * 2 + 2880 * 2)
    # x past one window: both paths refuse
    huge_t = (1 << 31) // (2880 * 4) + 1
    for path in (0, 1):
        assert lib.moe_mxfp4_workspace_bytes(ctypes.byref(big), huge_t, ctypes.byref(_opts(expert_path=path))) == 0
        assert _fwd(lib, big, T=huge_t, opts=_opts(expert_path=path)) == SHAPE
    # routing only: the grouping is always the routed one
    assert lib.moe_mxfp4_route(ctypes.byref(big), P, 4096, ctypes.byref(_opts(expert_path=7)), None, None, None,
                               None, None, None, P, 0, None) == WS


def test_workspace_bytes_grows_with_tokens(lib):
    L = _layer(E=32, H=2880, I=2880, top_k=4)
    o = _opts()
    a = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 64, ctypes.byref(o))
    b = lib.moe_mxfp4_workspace_bytes(ctypes.byref(L), 4096, ctypes.byref(o))
    assert 0 < a < b
    # dominated by the per-slot intermediate h and the expert outputs Y (both
    # bf16 with bf16 activations)
    assert b >= 4096 * 4 * (2880 * 2 + 2880 * 2)
    f = lib.moe_mxfp4_workspace_bytes(ctypes.byref(_layer(E=32, H=2880, I=2880, top_k=4, param_dtype=0)), 4096,
                                      ctypes.byref(_opts(act_dtype=0)))
    assert f >= 4096 * 4 * (2880 * 4 + 2880 * 4)  # fp32 activations: fp32 h and Y


def test_route_and_calibrate_validation(lib):
    L = _layer()
    o = _opts()
    r = lib.moe_mxfp4_route(ctypes.byref(_layer(H=36)), P, 8, ctypes.byref(o), P, P, P, P, P, P, P, 1 << 30, None)
    assert r == SHAPE
    r = lib.moe_mxfp4_route(ctypes.byref(L), P, 8, ctypes.byref(o), P + 4, P, P, P, P, P, P, 1 << 30, None)
    assert r == ALIGN
    r = lib.moe_mxfp4_route(ctypes.byref(L), P, 8, ctypes.byref(o), P, P, P, P, P, P, P, 16, None)
    assert r == WS
    assert lib.moe_mxfp4_route(ctypes.byref(L), P, 0, ctypes.byref(o), None, None, None, None, None, None, None, 0,
                               None) == OK
    assert lib.moe_mxfp4_calibrate_fp8(ctypes.byref(_layer(param_dtype=0)), P, 8, P, P, 1 << 30, None) == DTYPE
    assert lib.moe_mxfp4_calibrate_fp8(ctypes.byref(L), P, 0, P, P, 1 << 30, None) == SHAPE
    assert lib.moe_mxfp4_calibrate_fp8(ctypes.byref(L), P, 8, None, P, 1 << 30, None) == NULL


def test_binding_raises_on_bad_status(lib):
    with pytest.raises(mx.MxmoeError) as ei:
        B._check(SHAPE)
    assert ei.value.status == SHAPE and "multiple of 32" in str(ei.value)


def test_binding_has_no_cpu_fallback(tmp_path):
    # loading a missing library raises instead of computing anything elsewhere
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(OSError):
            B.load_library(str(tmp_path / "nope.so"))
    finally:
        B._lib = saved


def test_linear_validation(lib):
    s = None

    def call(x=P, T=8, K=64, wb=P, wsc=P, layout=0, bias=None, N=64, act=1, out=P, ws=P, ws_bytes=1 << 20):
        return lib.mxfp4_linear(x, T, K, wb, wsc, layout, bias, N, act, out, ws, ws_bytes, s)

    assert call(K=48) == SHAPE        # contracting dim not a multiple of 32 ("a clear error")
    assert call(K=0) == SHAPE
    assert call(N=40) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(act=3) == DTYPE
    assert call(layout=5) == VALUE
    assert call(wb=None) == NULL
    assert call(x=P + 2) == ALIGN
    assert call(bias=P + 8) == ALIGN
    assert call(T=0, x=None, out=None, ws=None) == OK  # empty batch: no-op
    need = lib.mxfp4_linear_workspace_bytes(8, 64, 1)
    assert need > 0
    assert call(ws_bytes=need - 1) == WS
    assert lib.mxfp4_linear_workspace_bytes(8, 64, 7) == 0


def test_fp8_linear_validation(lib):
    n = ctypes.c_int64(0)
    assert lib.fp8_tiled_bytes(64, 128, ctypes.byref(n)) == OK and n.value == 4 * 1 * 2048
    assert lib.fp8_tiled_bytes(96, 160, ctypes.byref(n)) == OK and n.value == 8 * 2 * 2048  # padded N and K
    assert lib.fp8_tiled_bytes(64, 48, ctypes.byref(n)) == SHAPE
    assert lib.fp8_tiled_bytes(0, 64, ctypes.byref(n)) == SHAPE
    assert lib.fp8_tiled_bytes(64, 64, None) == NULL
    assert lib.fp8_tile(P, 64, 48, P, None) == SHAPE
    assert lib.fp8_tile(None, 64, 64, P, None) == NULL
    assert lib.fp8_tile(P + 4, 64, 64, P, None) == ALIGN

    def call(T=8, K=64, N=64, x=P, w=P, w_scale=1.0, x_scale=1.0, bias=None, out=P, ws=P, ws_bytes=1 << 30):
        return lib.fp8_linear(x, T, K, w, w_scale, x_scale, bias, N, out, ws, ws_bytes, None)

    assert call(K=48) == SHAPE
    assert call(N=40) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(w_scale=0.0) == VALUE
    assert call(x_scale=float("inf")) == VALUE
    assert call(x_scale=float("nan")) == VALUE
    assert call(x_scale=1e-40) == VALUE  # 1 / x_scale overflows fp32
    assert call(x=None) == NULL
    assert call(w=None) == NULL
    assert call(bias=P + 2) == ALIGN
    assert call(out=P + 8) == ALIGN
    assert call(T=0, x=None, out=None, ws=None) == OK  # empty batch: no-op
    need = lib.fp8_linear_workspace_bytes(8, 64, 64)
    assert need >= 8 * 64  # holds x's FP8 codes
    assert call(ws_bytes=need - 1) == WS
    assert lib.fp8_linear_workspace_bytes(8, 48, 64) == 0
    assert lib.fp8_linear_workspace_bytes(-1, 64, 64) == 0


def _int8_layer(**kw):
    d = dict(E=8, H=64, I=64, top_k=2, gate_up_w=P, gate_up_scale=P, gate_up_bias=P, down_w=P, down_scale=P,
             down_bias=P, router_w=P, router_b=P)
    d.update(kw)
    return B.Int8Layer(**d)


def test_int8_validation(lib):
    n = ctypes.c_int64(0)
    assert lib.int8_tiled_bytes(3, 96, 160, ctypes.byref(n)) == OK and n.value == 3 * 8 * 2 * 2048
    assert lib.int8_tiled_bytes(1, 96, 48, ctypes.byref(n)) == SHAPE
    assert lib.int8_tiled_bytes(1, 96, 64, None) == NULL
    assert lib.int8_tile(P, 1, 64, 40, P, None) == SHAPE
    assert lib.int8_tile(None, 1, 64, 64, P, None) == NULL
    assert lib.int8_tile(P, 1, 64, 64, P + 1, None) == ALIGN
    assert lib.int8_tile(None, 0, 64, 64, None, None) == OK  # no matrices: no-op

    def fwd(L, T=8, x=P, out=P, idx=None, w=None, ws=P, ws_bytes=1 << 30):
        return lib.moe_int8_forward(ctypes.byref(L), x, T, out, idx, w, ws, ws_bytes, None)

    assert fwd(_int8_layer(H=48)) == SHAPE
    assert fwd(_int8_layer(top_k=9)) == SHAPE
    assert fwd(_int8_layer(E=0)) == SHAPE
    assert fwd(_int8_layer(down_scale=None)) == NULL
    assert fwd(_int8_layer(router_b=P + 2)) == ALIGN
    assert fwd(_int8_layer(), T=-1) == SHAPE
    assert fwd(_int8_layer(), T=0, x=None, out=None, ws=None) == OK
    assert fwd(_int8_layer(), x=None) == NULL
    assert fwd(_int8_layer(), idx=P + 4) == ALIGN
    L = _int8_layer()
    need = lib.moe_int8_workspace_bytes(ctypes.byref(L), 8)
    # routing tables, h and Y in bf16, x and h as int8 with one fp32 scale per row
    assert need >= 8 * 2 * (64 * 2 + 64 * 2) + 8 * 64 + 8 * 2 * 64
    assert fwd(L, ws_bytes=need - 1) == WS
    assert lib.moe_int8_workspace_bytes(ctypes.byref(_int8_layer(I=40)), 8) == 0


def test_binding_rejects_host_tensors(lib):
    """The Python binding refuses CPU tensors before any library call: every
    pointer the kernels receive must be device memory."""
    import torch

    blocks = torch.zeros((2, 1, 16), dtype=torch.uint8)
    scales = torch.zeros((2, 1), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensors"):
        mx.mxfp4_unpack(blocks, scales)
    with pytest.raises(ValueError, match="GPU tensors"):
        mx.mxfp4_pack(torch.zeros((2, 32), dtype=torch.bfloat16))
