"""MXFP4 mixture-of-experts layer for AMD MI355X (gfx950).

The computation lives in libmxmoe.so (hand-written HIP, C ABI in
include/mxmoe.h); this package only loads it and marshals torch tensors.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    FP8Linear,
    ForwardPlan,
    LAYOUT_ROWS,
    LAYOUT_TILED,
    LIB_PATH,
    MoEInt8Weights,
    MoEWeights,
    MXFP4Linear,
    MxmoeError,
    PATH_DENSE,
    PATH_ROUTED,
    alloc_workspace,
    fp8_linear,
    fp8_linear_workspace_bytes,
    fp8_tile,
    fp8_tiled_bytes,
    int8_tile,
    moe_int8_forward,
    moe_int8_workspace_bytes,
    load_library,
    moe_mxfp4_calibrate_fp8,
    moe_mxfp4_forward,
    moe_mxfp4_route,
    mxfp4_linear,
    mxfp4_linear_workspace_bytes,
    mxfp4_pack,
    mxfp4_tile,
    mxfp4_tiled_bytes,
    mxfp4_unpack,
    workspace_bytes,
)
