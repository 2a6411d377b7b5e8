"""Python binding of libmxmoe.so: argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch
tensors into device pointers, sizes and the current HIP stream, calls the
C ABI declared in include/mxmoe.h and raises on a non-zero status.  There is
no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxmoe.so")

MXMOE_F32 = 0
MXMOE_BF16 = 1
LAYOUT_ROWS = 0
LAYOUT_TILED = 1

STATUS_NAMES = {
    0: "MXMOE_OK",
    1: "MXMOE_ERR_NULL",
    2: "MXMOE_ERR_ALIGN",
    3: "MXMOE_ERR_SHAPE",
    4: "MXMOE_ERR_DTYPE",
    5: "MXMOE_ERR_WORKSPACE",
    6: "MXMOE_ERR_UNSUPPORTED",
    7: "MXMOE_ERR_HIP",
    8: "MXMOE_ERR_VALUE",
}

EXPORTED = (
    "mxmoe_status_string",
    "mxmoe_version",
    "mxfp4_unpack",
    "mxfp4_pack",
    "mxfp4_tiled_bytes",
    "mxfp4_tile",
    "mxfp4_linear_workspace_bytes",
    "mxfp4_linear",
    "fp8_tiled_bytes",
    "fp8_tile",
    "fp8_linear_workspace_bytes",
    "fp8_linear",
    "int8_tiled_bytes",
    "int8_tile",
    "moe_int8_workspace_bytes",
    "moe_int8_forward",
    "moe_mxfp4_workspace_bytes",
    "moe_mxfp4_forward",
    "moe_mxfp4_forward_noalloc",
    "moe_mxfp4_route",
    "moe_mxfp4_calibrate_fp8",
)


class MxmoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Layer(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("param_dtype", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
        ("gate_up_blocks", ctypes.c_void_p),
        ("gate_up_scales", ctypes.c_void_p),
        ("gate_up_bias", ctypes.c_void_p),
        ("down_blocks", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("down_bias", ctypes.c_void_p),
        ("router_w", ctypes.c_void_p),
        ("router_b", ctypes.c_void_p),
    ]


class Int8Layer(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("gate_up_w", ctypes.c_void_p),
        ("gate_up_scale", ctypes.c_void_p),
        ("gate_up_bias", ctypes.c_void_p),
        ("down_w", ctypes.c_void_p),
        ("down_scale", ctypes.c_void_p),
        ("down_bias", ctypes.c_void_p),
        ("router_w", ctypes.c_void_p),
        ("router_b", ctypes.c_void_p),
    ]


class FwdOpts(ctypes.Structure):
    _fields_ = [
        ("act_dtype", ctypes.c_int32),
        ("fp8_act", ctypes.c_int32),
        ("x_scale", ctypes.c_float),
        ("h_scale", ctypes.c_float),
        ("topk_idx_out", ctypes.c_void_p),
        ("topk_w_out", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
        ("expert_path", ctypes.c_int32),
    ]


# mxmoe_path_t
PATH_ROUTED, PATH_DENSE = 0, 1

STAGE_EVENTS = 7
STAGES = ("router", "grouping", "quant_fp8", "gate_up_swiglu", "down", "combine")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmxmoe.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with `python -m mxfp4_quantized_moe_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mxmoe_status_string.restype = ctypes.c_char_p
    lib.mxmoe_status_string.argtypes = [i32]
    lib.mxmoe_version.restype = i32
    lib.mxmoe_version.argtypes = []
    lib.mxfp4_unpack.restype = i32
    lib.mxfp4_unpack.argtypes = [vp, vp, i64, i64, vp, i32, vp]
    lib.mxfp4_pack.restype = i32
    lib.mxfp4_pack.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    lib.mxfp4_tiled_bytes.restype = i32
    lib.mxfp4_tiled_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.mxfp4_tile.restype = i32
    lib.mxfp4_tile.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
    lib.mxfp4_linear_workspace_bytes.restype = sz
    lib.mxfp4_linear_workspace_bytes.argtypes = [i64, i64, i32]
    lib.mxfp4_linear.restype = i32
    lib.mxfp4_linear.argtypes = [vp, i64, i64, vp, vp, i32, vp, i64, i32, vp, vp, sz, vp]
    f32 = ctypes.c_float
    lib.fp8_tiled_bytes.restype = i32
    lib.fp8_tiled_bytes.argtypes = [i64, i64, ctypes.POINTER(i64)]
    lib.fp8_tile.restype = i32
    lib.fp8_tile.argtypes = [vp, i64, i64, vp, vp]
    lib.fp8_linear_workspace_bytes.restype = sz
    lib.fp8_linear_workspace_bytes.argtypes = [i64, i64, i64]
    lib.fp8_linear.restype = i32
    lib.fp8_linear.argtypes = [vp, i64, i64, vp, f32, f32, vp, i64, vp, vp, sz, vp]
    lib.int8_tiled_bytes.restype = i32
    lib.int8_tiled_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    lib.int8_tile.restype = i32
    lib.int8_tile.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.moe_int8_workspace_bytes.restype = sz
    lib.moe_int8_workspace_bytes.argtypes = [ctypes.POINTER(Int8Layer), i64]
    lib.moe_int8_forward.restype = i32
    lib.moe_int8_forward.argtypes = [ctypes.POINTER(Int8Layer), vp, i64, vp, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_workspace_bytes.restype = sz
    lib.moe_mxfp4_workspace_bytes.argtypes = [ctypes.POINTER(Layer), i64, ctypes.POINTER(FwdOpts)]
    lib.moe_mxfp4_forward.restype = i32
    lib.moe_mxfp4_forward.argtypes = [ctypes.POINTER(Layer), vp, i64, vp, ctypes.POINTER(FwdOpts), vp, sz, vp]
    lib.moe_mxfp4_forward_noalloc.restype = i32
    lib.moe_mxfp4_forward_noalloc.argtypes = [ctypes.POINTER(Layer), vp, i64, vp, ctypes.POINTER(FwdOpts), vp]
    lib.moe_mxfp4_route.restype = i32
    lib.moe_mxfp4_route.argtypes = [ctypes.POINTER(Layer), vp, i64, ctypes.POINTER(FwdOpts),
                                    vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_calibrate_fp8.restype = i32
    lib.moe_mxfp4_calibrate_fp8.argtypes = [ctypes.POINTER(Layer), vp, i64, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().mxmoe_status_string(status).decode()
        raise MxmoeError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:  # the kernels dereference every pointer on the GPU
        raise ValueError("tensors passed to the library must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MXMOE_BF16
    if dt == torch.float32:
        return MXMOE_F32
    raise ValueError(f"unsupported dtype {dt}")


# Shape checks done here, before any pointer reaches the library: the C ABI
# takes sizes, not shapes, so a tensor smaller than the sizes say would be
# read or written past its end by the kernels.


def _expect(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, min_numel: Optional[int] = None) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if min_numel is not None and (t.dim() != 1 or t.numel() < min_numel):
        raise ValueError(f"{name} must be a flat tensor of at least {min_numel} elements, got {tuple(t.shape)}")


def _expect_same_device(*ts: Optional[torch.Tensor]) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors passed to one call must share a device, got {sorted(map(str, devs))}")


def _expect_out(out: torch.Tensor, shape, dtype, name: str = "out") -> None:
    _expect(out, name, shape, dtype)


# ---------------------------------------------------------------- codec


def mxfp4_unpack(blocks: torch.Tensor, scales: torch.Tensor, dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(..., nb, 16) uint8 blocks + (..., nb) uint8 scales -> (..., nb*32)."""
    if blocks.dim() < 2 or blocks.shape[-1] != 16:
        raise ValueError(f"blocks must be (..., nb, 16), got {tuple(blocks.shape)}")
    nb = blocks.shape[-2]
    lead = tuple(blocks.shape[:-2])
    _expect(blocks, "blocks", dtype=torch.uint8)
    _expect(scales, "scales", lead + (nb,), torch.uint8)
    rows = 1
    for d in lead:
        rows *= d
    if out is None:
        out = torch.empty(lead + (nb * 32,), dtype=dtype, device=blocks.device)
    _expect_out(out, lead + (nb * 32,), out.dtype)
    _dtype_code(out.dtype)
    _expect_same_device(blocks, scales, out)
    _check(load_library().mxfp4_unpack(_ptr(blocks), _ptr(scales), rows, nb * 32, _ptr(out),
                                       _dtype_code(out.dtype), _stream(blocks.device)))
    return out


def mxfp4_pack(w: torch.Tensor):
    """(..., K) bf16/fp32 -> (blocks (..., K/32, 16) uint8, scales (..., K/32) uint8)."""
    if w.dim() < 1:
        raise ValueError("w must have a contracting dimension")
    _dtype_code(w.dtype)
    K = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = 1
    for d in lead:
        rows *= d
    blocks = torch.empty(lead + (max(K // 32, 0), 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty(lead + (max(K // 32, 0),), dtype=torch.uint8, device=w.device)
    _check(load_library().mxfp4_pack(_ptr(w), _dtype_code(w.dtype), rows, K, _ptr(blocks), _ptr(scales),
                                     _stream(w.device)))
    return blocks, scales


def mxfp4_tiled_bytes(mats: int, rows: int, k: int):
    """Byte sizes (blocks, scales) of the tiled copy of `mats` (rows, k) MXFP4 matrices."""
    bb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(load_library().mxfp4_tiled_bytes(mats, rows, k, ctypes.byref(bb), ctypes.byref(sb)))
    return int(bb.value), int(sb.value)


def mxfp4_tile(blocks: torch.Tensor, scales: torch.Tensor):
    """(mats, rows, nb, 16) blocks + (mats, rows, nb) scales in row order ->
    flat uint8 (tiled_blocks, tiled_scales) in the tiled order of mxmoe.h."""
    if blocks.dim() != 4 or blocks.shape[-1] != 16:
        raise ValueError(f"blocks must be (mats, rows, nb, 16), got {tuple(blocks.shape)}")
    mats, rows, nb = (int(d) for d in blocks.shape[:3])
    _expect(blocks, "blocks", dtype=torch.uint8)
    _expect(scales, "scales", (mats, rows, nb), torch.uint8)
    _expect_same_device(blocks, scales)
    bb, sb = mxfp4_tiled_bytes(mats, rows, nb * 32)
    tb = torch.empty(max(bb, 16), dtype=torch.uint8, device=blocks.device)[:bb]
    ts = torch.empty(max(sb, 16), dtype=torch.uint8, device=blocks.device)[:sb]
    _check(load_library().mxfp4_tile(_ptr(blocks), _ptr(scales), mats, rows, nb * 32, _ptr(tb), _ptr(ts),
                                     _stream(blocks.device)))
    return tb, ts


# ----------------------------------------------------------- dense layer


@dataclass
class MXFP4Linear:
    """A weight-only MXFP4 dense layer y = x W^T + b (see include/mxmoe.h).
    blocks/scales: (N, K/32, 16) / (N, K/32) in row order, or the flat
    outputs of mxfp4_tile with layout LAYOUT_TILED."""

    blocks: torch.Tensor
    scales: torch.Tensor
    N: int
    K: int
    bias: Optional[torch.Tensor] = None  # (N,) in the activation dtype
    layout: int = LAYOUT_ROWS

    @staticmethod
    def from_rows(blocks: torch.Tensor, scales: torch.Tensor, bias: Optional[torch.Tensor] = None) -> "MXFP4Linear":
        return MXFP4Linear(blocks, scales, int(blocks.shape[0]), int(blocks.shape[1]) * 32, bias)

    def tiled(self) -> "MXFP4Linear":
        if self.layout == LAYOUT_TILED:
            return self
        tb, ts = mxfp4_tile(self.blocks.reshape(1, self.N, self.K // 32, 16), self.scales.reshape(1, self.N, self.K // 32))
        return MXFP4Linear(tb, ts, self.N, self.K, self.bias, LAYOUT_TILED)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        return mxfp4_linear(x, self, out=out, workspace=workspace)

    def validate(self, act_dtype: torch.dtype) -> None:
        """Tensor shapes and dtypes against N, K (ValueError on a mismatch)."""
        if self.layout == LAYOUT_TILED:
            bb, sb = mxfp4_tiled_bytes(1, self.N, self.K)
            _expect(self.blocks, "blocks", dtype=torch.uint8, min_numel=bb)
            _expect(self.scales, "scales", dtype=torch.uint8, min_numel=sb)
        elif self.layout == LAYOUT_ROWS:
            _expect(self.blocks, "blocks", (self.N, self.K // 32, 16), torch.uint8)
            _expect(self.scales, "scales", (self.N, self.K // 32), torch.uint8)
        else:
            raise ValueError(f"unknown layout {self.layout}")
        if self.bias is not None:
            _expect(self.bias, "bias", (self.N,), act_dtype)
        _expect_same_device(self.blocks, self.scales, self.bias)


def mxfp4_linear_workspace_bytes(T: int, N: int, act_dtype: torch.dtype) -> int:
    return int(load_library().mxfp4_linear_workspace_bytes(T, N, _dtype_code(act_dtype)))


def mxfp4_linear(x: torch.Tensor, layer: MXFP4Linear, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W^T + b for x (T, K) in bf16 or fp32; returns (T, N)."""
    if x.dim() != 2 or int(x.shape[1]) != layer.K:
        raise ValueError(f"x must be (T, {layer.K}), got {tuple(x.shape)}")
    _dtype_code(x.dtype)
    layer.validate(x.dtype)
    T = int(x.shape[0])
    if out is None:
        out = torch.empty((T, layer.N), dtype=x.dtype, device=x.device)
    _expect_out(out, (T, layer.N), x.dtype)
    _expect_same_device(x, layer.blocks, out, workspace)
    if workspace is None:
        n = mxfp4_linear_workspace_bytes(T, layer.N, x.dtype)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    _check(load_library().mxfp4_linear(_ptr(x), T, int(x.shape[1]), _ptr(layer.blocks), _ptr(layer.scales),
                                       layer.layout, _ptr(layer.bias), layer.N, _dtype_code(x.dtype), _ptr(out),
                                       _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


# ------------------------------------------------------- dense FP8 layer


def fp8_tiled_bytes(N: int, K: int) -> int:
    n = ctypes.c_int64(0)
    _check(load_library().fp8_tiled_bytes(N, K, ctypes.byref(n)))
    return int(n.value)


def fp8_tile(w: torch.Tensor) -> torch.Tensor:
    """(N, K) uint8 e4m3 codes (row-major, device) -> the tiled FP8 order."""
    if w.dim() != 2:
        raise ValueError(f"w must be (N, K), got {tuple(w.shape)}")
    _expect(w, "w", dtype=torch.uint8)
    N, K = int(w.shape[0]), int(w.shape[1])
    out = torch.empty(fp8_tiled_bytes(N, K), dtype=torch.uint8, device=w.device)
    _check(load_library().fp8_tile(_ptr(w.contiguous()), N, K, _ptr(out), _stream(w.device)))
    return out


@dataclass
class FP8Linear:
    """A dense FP8 E4M3 layer with static per-tensor scales (W8A8):
    y = (q(x) q(W)^T) * (x_scale * w_scale) + b, see include/mxmoe.h.
    w_tiled is fp8_tile's output; bias (N,) bf16 or None."""

    w_tiled: torch.Tensor
    N: int
    K: int
    w_scale: float
    x_scale: float
    bias: Optional[torch.Tensor] = None

    @staticmethod
    def from_codes(w: torch.Tensor, w_scale: float, x_scale: float,
                   bias: Optional[torch.Tensor] = None) -> "FP8Linear":
        return FP8Linear(fp8_tile(w), int(w.shape[0]), int(w.shape[1]), float(w_scale), float(x_scale), bias)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        return fp8_linear(x, self, out=out, workspace=workspace)

    def validate(self) -> None:
        """Tensor shapes and dtypes against N, K (ValueError on a mismatch)."""
        _expect(self.w_tiled, "w_tiled", dtype=torch.uint8, min_numel=fp8_tiled_bytes(self.N, self.K))
        if self.bias is not None:
            _expect(self.bias, "bias", (self.N,), torch.bfloat16)
        _expect_same_device(self.w_tiled, self.bias)


def fp8_linear_workspace_bytes(T: int, K: int, N: int) -> int:
    return int(load_library().fp8_linear_workspace_bytes(T, K, N))


def fp8_linear(x: torch.Tensor, layer: FP8Linear, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x (T, K) bf16 -> (T, N) bf16."""
    _expect(x, "x", dtype=torch.bfloat16)
    if x.dim() != 2 or int(x.shape[1]) != layer.K:
        raise ValueError(f"x must be (T, {layer.K}), got {tuple(x.shape)}")
    layer.validate()
    T = int(x.shape[0])
    if out is None:
        out = torch.empty((T, layer.N), dtype=torch.bfloat16, device=x.device)
    _expect_out(out, (T, layer.N), torch.bfloat16)
    _expect_same_device(x, layer.w_tiled, out, workspace)
    if workspace is None:
        n = fp8_linear_workspace_bytes(T, layer.K, layer.N)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    _check(load_library().fp8_linear(_ptr(x), T, int(x.shape[1]), _ptr(layer.w_tiled), layer.w_scale, layer.x_scale,
                                     _ptr(layer.bias), layer.N, _ptr(out), _ptr(workspace), workspace.numel(),
                                     _stream(x.device)))
    return out


# ----------------------------------------------------- int8 W8A8 layer


def int8_tile(w: torch.Tensor) -> torch.Tensor:
    """(mats, rows, k) int8 codes (device) -> the tiled 8-bit order (flat)."""
    if w.dim() != 3:
        raise ValueError(f"w must be (mats, rows, k), got {tuple(w.shape)}")
    _expect(w, "w", dtype=torch.int8)
    mats, rows, k = (int(v) for v in w.shape)
    n = ctypes.c_int64(0)
    _check(load_library().int8_tiled_bytes(mats, rows, k, ctypes.byref(n)))
    out = torch.empty(int(n.value), dtype=torch.uint8, device=w.device)
    _check(load_library().int8_tile(_ptr(w.contiguous()), mats, rows, k, _ptr(out), _stream(w.device)))
    return out


@dataclass
class MoEInt8Weights:
    """Device tensors of one INT8 W8A8 MoE layer (see include/mxmoe.h); the
    two weights are int8_tile outputs (from_codes tiles them)."""

    gate_up_w: torch.Tensor      # tiled (E, 2I, H) int8 codes
    gate_up_scale: torch.Tensor  # (E, 2I) fp32
    gate_up_bias: torch.Tensor   # (E, 2I) bf16
    down_w: torch.Tensor         # tiled (E, H, I) int8 codes
    down_scale: torch.Tensor     # (E, H) fp32
    down_bias: torch.Tensor      # (E, H) bf16
    router_w: torch.Tensor       # (E, H) bf16
    router_b: torch.Tensor       # (E,) bf16
    top_k: int

    @staticmethod
    def from_codes(gate_up: torch.Tensor, gate_up_scale, gate_up_bias, down: torch.Tensor, down_scale, down_bias,
                   router_w, router_b, top_k: int) -> "MoEInt8Weights":
        return MoEInt8Weights(int8_tile(gate_up), gate_up_scale, gate_up_bias, int8_tile(down), down_scale,
                              down_bias, router_w, router_b, top_k)

    @property
    def E(self) -> int:
        return int(self.router_w.shape[0])

    @property
    def H(self) -> int:
        return int(self.router_w.shape[1])

    @property
    def I(self) -> int:  # noqa: E743
        return int(self.gate_up_bias.shape[1]) // 2

    def validate(self) -> None:
        """Every tensor's shape and dtype against E, H, I (ValueError on a
        mismatch): the library sizes its reads from those alone."""
        if self.router_w.dim() != 2 or self.gate_up_bias.dim() != 2 or self.gate_up_bias.shape[1] % 2:
            raise ValueError("router_w must be (E, H) and gate_up_bias (E, 2I)")
        E, H, I = self.E, self.H, self.I
        bf = torch.bfloat16
        n = ctypes.c_int64(0)
        _check(load_library().int8_tiled_bytes(E, 2 * I, H, ctypes.byref(n)))
        _expect(self.gate_up_w, "gate_up_w", dtype=torch.uint8, min_numel=int(n.value))
        _check(load_library().int8_tiled_bytes(E, H, I, ctypes.byref(n)))
        _expect(self.down_w, "down_w", dtype=torch.uint8, min_numel=int(n.value))
        _expect(self.gate_up_scale, "gate_up_scale", (E, 2 * I), torch.float32)
        _expect(self.gate_up_bias, "gate_up_bias", (E, 2 * I), bf)
        _expect(self.down_scale, "down_scale", (E, H), torch.float32)
        _expect(self.down_bias, "down_bias", (E, H), bf)
        _expect(self.router_w, "router_w", (E, H), bf)
        _expect(self.router_b, "router_b", (E,), bf)
        _expect_same_device(self.gate_up_w, self.gate_up_scale, self.gate_up_bias, self.down_w, self.down_scale,
                            self.down_bias, self.router_w, self.router_b)

    def descriptor(self) -> Int8Layer:
        return Int8Layer(E=self.E, H=self.H, I=self.I, top_k=self.top_k, gate_up_w=_ptr(self.gate_up_w),
                         gate_up_scale=_ptr(self.gate_up_scale), gate_up_bias=_ptr(self.gate_up_bias),
                         down_w=_ptr(self.down_w), down_scale=_ptr(self.down_scale), down_bias=_ptr(self.down_bias),
                         router_w=_ptr(self.router_w), router_b=_ptr(self.router_b))


def moe_int8_workspace_bytes(layer: MoEInt8Weights, T: int) -> int:
    d = layer.descriptor()
    n = load_library().moe_int8_workspace_bytes(ctypes.byref(d), T)
    if n == 0 and T > 0:
        raise MxmoeError(3, "invalid int8 layer or token count")
    return int(n)


def moe_int8_forward(layer: MoEInt8Weights, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, topk_idx_out: Optional[torch.Tensor] = None,
                     topk_w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The INT8 W8A8 MoE layer on x (T, H) bf16; returns out (T, H) bf16."""
    layer.validate()
    _expect(x, "x", dtype=torch.bfloat16)
    if x.dim() != 2 or int(x.shape[1]) != layer.H:
        raise ValueError(f"x must be (T, {layer.H}), got {tuple(x.shape)}")
    T = int(x.shape[0])
    if out is None:
        out = torch.empty_like(x)
    _expect_out(out, (T, layer.H), torch.bfloat16)
    _check_topk_outs(topk_idx_out, topk_w_out, T, layer.top_k)
    _expect_same_device(x, layer.router_w, out, workspace, topk_idx_out, topk_w_out)
    if workspace is None:
        workspace = torch.empty(max(moe_int8_workspace_bytes(layer, T), 256), dtype=torch.uint8, device=x.device)
    d = layer.descriptor()
    _check(load_library().moe_int8_forward(ctypes.byref(d), _ptr(x), T, _ptr(out), _ptr(topk_idx_out),
                                           _ptr(topk_w_out), _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


# ----------------------------------------------------------------- layer


@dataclass
class MoEWeights:
    """Device tensors of one MXFP4 MoE layer (see include/mxmoe.h).  With
    layout LAYOUT_TILED the four MXFP4 tensors are the flat outputs of
    mxfp4_tile; the shapes noted are those of LAYOUT_ROWS."""

    gate_up_blocks: torch.Tensor  # (E, 2I, H/32, 16) uint8
    gate_up_scales: torch.Tensor  # (E, 2I, H/32) uint8
    gate_up_bias: torch.Tensor  # (E, 2I)
    down_blocks: torch.Tensor  # (E, H, I/32, 16) uint8
    down_scales: torch.Tensor  # (E, H, I/32) uint8
    down_bias: torch.Tensor  # (E, H)
    router_w: torch.Tensor  # (E, H)
    router_b: torch.Tensor  # (E,)
    top_k: int
    layout: int = LAYOUT_ROWS

    @property
    def E(self) -> int:
        return int(self.router_w.shape[0])

    @property
    def H(self) -> int:
        return int(self.router_w.shape[1])

    @property
    def I(self) -> int:
        return int(self.gate_up_bias.shape[1]) // 2

    def tiled(self) -> "MoEWeights":
        """A copy of the layer with its MXFP4 tensors in the tiled order
        (the GEMM-friendly layout; a one-time step at load)."""
        if self.layout == LAYOUT_TILED:
            return self
        gb, gs = mxfp4_tile(self.gate_up_blocks, self.gate_up_scales)
        db, ds = mxfp4_tile(self.down_blocks, self.down_scales)
        return MoEWeights(gb, gs, self.gate_up_bias, db, ds, self.down_bias, self.router_w, self.router_b,
                          top_k=self.top_k, layout=LAYOUT_TILED)

    def validate(self) -> None:
        """Every tensor's shape and dtype against E, H, I and the layout
        (ValueError on a mismatch): the library sizes its reads from those
        alone.  Router and biases share one dtype (bf16 or fp32)."""
        if self.router_w.dim() != 2 or self.gate_up_bias.dim() != 2 or self.gate_up_bias.shape[1] % 2:
            raise ValueError("router_w must be (E, H) and gate_up_bias (E, 2I)")
        E, H, I = self.E, self.H, self.I
        pd = self.router_w.dtype
        _dtype_code(pd)
        _expect(self.router_b, "router_b", (E,), pd)
        _expect(self.gate_up_bias, "gate_up_bias", (E, 2 * I), pd)
        _expect(self.down_bias, "down_bias", (E, H), pd)
        u8 = torch.uint8
        if self.layout == LAYOUT_ROWS:
            if H % 32 or I % 32:
                raise ValueError(f"H and I must be multiples of 32, got {H}, {I}")
            _expect(self.gate_up_blocks, "gate_up_blocks", (E, 2 * I, H // 32, 16), u8)
            _expect(self.gate_up_scales, "gate_up_scales", (E, 2 * I, H // 32), u8)
            _expect(self.down_blocks, "down_blocks", (E, H, I // 32, 16), u8)
            _expect(self.down_scales, "down_scales", (E, H, I // 32), u8)
        elif self.layout == LAYOUT_TILED:
            gb, gs = mxfp4_tiled_bytes(E, 2 * I, H)
            db, ds = mxfp4_tiled_bytes(E, H, I)
            _expect(self.gate_up_blocks, "gate_up_blocks", dtype=u8, min_numel=gb)
            _expect(self.gate_up_scales, "gate_up_scales", dtype=u8, min_numel=gs)
            _expect(self.down_blocks, "down_blocks", dtype=u8, min_numel=db)
            _expect(self.down_scales, "down_scales", dtype=u8, min_numel=ds)
        else:
            raise ValueError(f"unknown layout {self.layout}")
        _expect_same_device(self.gate_up_blocks, self.gate_up_scales, self.gate_up_bias, self.down_blocks,
                            self.down_scales, self.down_bias, self.router_w, self.router_b)

    def descriptor(self) -> Layer:
        return Layer(
            E=self.E, H=self.H, I=self.I, top_k=self.top_k, param_dtype=_dtype_code(self.router_w.dtype),
            weight_layout=self.layout,
            gate_up_blocks=_ptr(self.gate_up_blocks), gate_up_scales=_ptr(self.gate_up_scales),
            gate_up_bias=_ptr(self.gate_up_bias), down_blocks=_ptr(self.down_blocks),
            down_scales=_ptr(self.down_scales), down_bias=_ptr(self.down_bias), router_w=_ptr(self.router_w),
            router_b=_ptr(self.router_b))


def _check_x(layer, x: torch.Tensor) -> int:
    """x must be (T, H) in the layer's parameter dtype; returns T."""
    layer.validate()
    if x.dim() != 2 or int(x.shape[1]) != layer.H:
        raise ValueError(f"x must be (T, {layer.H}), got {tuple(x.shape)}")
    if x.dtype != layer.router_w.dtype:
        raise ValueError(f"x must have the parameters' dtype {layer.router_w.dtype}, got {x.dtype}")
    return int(x.shape[0])


def _check_topk_outs(idx_out: Optional[torch.Tensor], w_out: Optional[torch.Tensor], T: int, k: int) -> None:
    if idx_out is not None:
        _expect(idx_out, "topk_idx_out", (T, k), torch.int32)
    if w_out is not None:
        _expect(w_out, "topk_w_out", (T, k), torch.float32)


def _opts(act_dtype: torch.dtype, fp8: bool, x_scale: float, h_scale: float, idx_out=None, w_out=None,
          stage_events=None, dense: bool = False) -> FwdOpts:
    return FwdOpts(act_dtype=_dtype_code(act_dtype), fp8_act=1 if fp8 else 0, x_scale=x_scale, h_scale=h_scale,
                   topk_idx_out=_ptr(idx_out), topk_w_out=_ptr(w_out),
                   stage_events=ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None,
                   expert_path=PATH_DENSE if dense else PATH_ROUTED)


def workspace_bytes(layer: MoEWeights, T: int, act_dtype: torch.dtype, fp8: bool = False,
                    dense: bool = False) -> int:
    d = layer.descriptor()
    o = _opts(act_dtype, fp8, 1.0, 1.0, dense=dense)
    n = load_library().moe_mxfp4_workspace_bytes(ctypes.byref(d), T, ctypes.byref(o))
    if n == 0 and T > 0:
        raise MxmoeError(3, "invalid layer or token count")
    return int(n)


def alloc_workspace(layer: MoEWeights, T: int, act_dtype: torch.dtype, fp8: bool = False,
                    dense: bool = False) -> torch.Tensor:
    n = workspace_bytes(layer, T, act_dtype, fp8, dense)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=layer.router_w.device)


def moe_mxfp4_forward(layer: MoEWeights, x: torch.Tensor, fp8: bool = False, x_scale: float = 1.0,
                      h_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, topk_idx_out: Optional[torch.Tensor] = None,
                      topk_w_out: Optional[torch.Tensor] = None, stage_events=None,
                      dense: bool = False) -> torch.Tensor:
    """The MXFP4 MoE layer on x (T, H); returns out (T, H).

    dense: every token through every expert (MXMOE_PATH_DENSE) instead of
    its top_k; the combine is the same.
    stage_events: optional ctypes array of STAGE_EVENTS hipEvent_t handles
    (see include/mxmoe.h) recorded around the stages on the current stream."""
    T = _check_x(layer, x)
    if out is None:
        out = torch.empty_like(x)
    _expect_out(out, (T, layer.H), x.dtype)
    _check_topk_outs(topk_idx_out, topk_w_out, T, layer.top_k)
    _expect_same_device(x, layer.router_w, out, workspace, topk_idx_out, topk_w_out)
    if workspace is None:
        workspace = alloc_workspace(layer, T, x.dtype, fp8, dense)
    d = layer.descriptor()
    o = _opts(x.dtype, fp8, x_scale, h_scale, topk_idx_out, topk_w_out, stage_events, dense)
    _check(load_library().moe_mxfp4_forward(ctypes.byref(d), _ptr(x), T, _ptr(out), ctypes.byref(o),
                                            _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


# Size of the library's own scratch array used by moe_mxfp4_forward_noalloc
# (MXMOE_NOALLOC_SCRATCH_BYTES in include/mxmoe.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_mxfp4_forward_noalloc(layer: MoEWeights, x: torch.Tensor, out: torch.Tensor, fp8: bool = False,
                              x_scale: float = 1.0, h_scale: float = 1.0,
                              topk_idx_out: Optional[torch.Tensor] = None,
                              topk_w_out: Optional[torch.Tensor] = None, dense: bool = False) -> torch.Tensor:
    """moe_mxfp4_forward on the library's fixed scratch array instead of a
    workspace: nothing is allocated (out is the caller's).  Batches whose
    workspace_bytes exceed NOALLOC_SCRATCH_BYTES raise MXMOE_ERR_WORKSPACE;
    calls that may overlap on one GPU must be ordered by the caller."""
    T = _check_x(layer, x)
    _expect_out(out, (T, layer.H), x.dtype)
    _check_topk_outs(topk_idx_out, topk_w_out, T, layer.top_k)
    _expect_same_device(x, layer.router_w, out, topk_idx_out, topk_w_out)
    d = layer.descriptor()
    o = _opts(x.dtype, fp8, x_scale, h_scale, topk_idx_out, topk_w_out, None, dense)
    _check(load_library().moe_mxfp4_forward_noalloc(ctypes.byref(d), _ptr(x), T, _ptr(out), ctypes.byref(o),
                                                    _stream(x.device)))
    return out


class ForwardPlan:
    """A prepared moe_mxfp4_forward call for a loop that repeats it on the
    same tensors (a serving or benchmark loop): the tensors are checked and
    the descriptor is built once; each call then only passes the stored
    arguments and the current stream to the library.  The tensors must keep
    their shapes and storage for the plan's lifetime (their contents may
    change between calls)."""

    def __init__(self, layer: MoEWeights, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, fp8: bool = False, x_scale: float = 1.0,
                 h_scale: float = 1.0, topk_idx_out: Optional[torch.Tensor] = None,
                 topk_w_out: Optional[torch.Tensor] = None, dense: bool = False):
        T = _check_x(layer, x)
        if out is None:
            out = torch.empty_like(x)
        _expect_out(out, (T, layer.H), x.dtype)
        _check_topk_outs(topk_idx_out, topk_w_out, T, layer.top_k)
        if workspace is None:
            workspace = alloc_workspace(layer, T, x.dtype, fp8, dense)
        _expect_same_device(x, layer.router_w, out, workspace, topk_idx_out, topk_w_out)
        self.layer, self.x, self.out, self.workspace = layer, x, out, workspace
        self._keep = (topk_idx_out, topk_w_out)
        self._d = layer.descriptor()
        self._o = _opts(x.dtype, fp8, x_scale, h_scale, topk_idx_out, topk_w_out, None, dense)
        self._dev = x.device
        self._fn = load_library().moe_mxfp4_forward
        self._args = (ctypes.byref(self._d), _ptr(x), T, _ptr(out), ctypes.byref(self._o), _ptr(workspace),
                      workspace.numel())

    def __call__(self, stage_events=None) -> torch.Tensor:
        """Enqueue the forward on the current stream; returns out."""
        if stage_events is not None:
            self._o.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
        try:
            _check(self._fn(*self._args, _stream(self._dev)))
        finally:
            if stage_events is not None:
                self._o.stage_events = None
        return self.out


def moe_mxfp4_route(layer: MoEWeights, x: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Routing only: returns (idx, w, counts, offsets, sorted_slots, slot_pos)."""
    T = _check_x(layer, x)
    _expect_same_device(x, layer.router_w, workspace)
    k, E = layer.top_k, layer.E
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sorted_slots = torch.empty((T * k,), dtype=torch.int32, device=dev)
    pos = torch.empty((T * k,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(layer, T, x.dtype)
    d = layer.descriptor()
    o = _opts(x.dtype, False, 1.0, 1.0)
    _check(load_library().moe_mxfp4_route(ctypes.byref(d), _ptr(x), T, ctypes.byref(o), _ptr(idx), _ptr(w),
                                          _ptr(counts), _ptr(offsets), _ptr(sorted_slots), _ptr(pos),
                                          _ptr(workspace), workspace.numel(), _stream(dev)))
    return idx, w, counts, offsets, sorted_slots, pos


def moe_mxfp4_calibrate_fp8(layer: MoEWeights, x_calib: torch.Tensor,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Static FP8 scales (s_x, s_h) from a bf16 calibration batch, as a device float[2]."""
    T = _check_x(layer, x_calib)
    if x_calib.dtype != torch.bfloat16:
        raise ValueError("the calibration batch must be bf16")
    _expect_same_device(x_calib, layer.router_w, workspace)
    scales = torch.empty((4,), dtype=torch.float32, device=x_calib.device)
    if workspace is None:
        workspace = alloc_workspace(layer, T, torch.bfloat16)
    d = layer.descriptor()
    _check(load_library().moe_mxfp4_calibrate_fp8(ctypes.byref(d), _ptr(x_calib), T, _ptr(scales),
                                                  _ptr(workspace), workspace.numel(), _stream(x_calib.device)))
    return scales[:2]
