"""Seeded synthetic inputs for the MXFP4 mixture-of-experts layer.

This module only draws random numbers and stores them in the layouts the
layer consumes.  It holds none of the layer's arithmetic (no decode, no
routing, no quantisation), so both the CPU oracle and the HIP path can take
their inputs from it without sharing any of the method's code.

Shapes follow the GPT-OSS expert layout described on the KerasFormers
"mxfp4" page, section "As GPT-OSS's native format": gate_up_proj is
(E, 2I, H) and down_proj is (E, H, I), each stored as uint8 nibble-pair
blocks (rows, K/32, 16) plus one uint8 e8m0 scale per 32-value block, with
full-precision biases.  Rows 2i and 2i+1 of gate_up are gate_i and up_i.

Representation: uint8 arrays for blocks and scales; float32 arrays for fp32
tensors; uint16 arrays holding raw bfloat16 bit patterns for bf16 tensors.
bf16 values are drawn in float64, cast to float32 by numpy, then rounded to
bfloat16 by torch's CPU cast (round-to-nearest-even); that cast is input
preparation, not part of the layer.

Draw order within one layer (one numpy PCG64 generator): gate_up blocks,
gate_up scales, gate_up bias, down blocks, down scales, down bias, router
weight, router bias, x.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns to float32 (exact: a bit shift)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _real(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.normal(0.0, std, size=shape).astype(np.float32)
    return _to_bf16_bits(a) if dtype == BF16 else a


@dataclass
class MoELayer:
    """One MXFP4 MoE layer's parameters (host copies)."""

    E: int
    H: int
    I: int
    top_k: int
    gate_up_blocks: np.ndarray  # (E, 2I, H/32, 16) uint8
    gate_up_scales: np.ndarray  # (E, 2I, H/32) uint8
    gate_up_bias: np.ndarray  # (E, 2I) param dtype
    down_blocks: np.ndarray  # (E, H, I/32, 16) uint8
    down_scales: np.ndarray  # (E, H, I/32) uint8
    down_bias: np.ndarray  # (E, H) param dtype
    router_w: np.ndarray  # (E, H) param dtype
    router_b: np.ndarray  # (E,) param dtype
    param_dtype: str  # "bf16" | "f32"


@dataclass
class MoECase:
    name: str
    layer: MoELayer
    x: np.ndarray  # (T, H) act dtype
    act_dtype: str
    fp8: bool = False
    x_calib: Optional[np.ndarray] = None  # (Tc, H) act dtype, FP8 mode only
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.x.shape[0])


def make_layer(
    rng: np.random.Generator,
    E: int,
    H: int,
    I: int,
    top_k: int,
    param_dtype: str,
    scale_lo: int,
    scale_hi: int,
    bias_std: float,
    router_std: float,
    router_bias_std: float,
) -> MoELayer:
    """Draw one layer in the fixed order; scale bytes uniform on [lo, hi]."""
    assert H % 32 == 0 and I % 32 == 0
    gub = rng.integers(0, 256, size=(E, 2 * I, H // 32, 16), dtype=np.uint8)
    gus = rng.integers(scale_lo, scale_hi + 1, size=(E, 2 * I, H // 32), dtype=np.uint8)
    gubias = _real(rng, (E, 2 * I), bias_std, param_dtype)
    db = rng.integers(0, 256, size=(E, H, I // 32, 16), dtype=np.uint8)
    ds = rng.integers(scale_lo, scale_hi + 1, size=(E, H, I // 32), dtype=np.uint8)
    dbias = _real(rng, (E, H), bias_std, param_dtype)
    rw = _real(rng, (E, H), router_std, param_dtype)
    rb = _real(rng, (E,), router_bias_std, param_dtype)
    return MoELayer(E, H, I, top_k, gub, gus, gubias, db, ds, dbias, rw, rb, param_dtype)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------


def tiny(seed: int = 0, T: int = 8) -> MoECase:
    """E=4, top-2, H=I=64, T=8, all fp32; scales on [120, 126]."""
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, 4, 64, 64, 2, F32, 120, 126, 0.01, 0.1, 0.01)
    x = _real(rng, (T, 64), 1.0, F32)
    return MoECase("tiny_e4_k2_h64_t8_f32", layer, x, F32)


def decode_20b(T: int = 64, seed: int = 0) -> MoECase:
    """gpt-oss-20b-shaped decode: E=32, top-4, H=I=2880, bf16; T in {1, 8, 64}.

    x is drawn for 64 tokens and the first T rows are used, so the smaller
    decode batches are prefixes of the largest one."""
    assert 1 <= T <= 64
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, 32, 2880, 2880, 4, BF16, 120, 126, 0.01, 0.02, 0.01)
    x = _real(rng, (64, 2880), 1.0, BF16)[:T].copy()
    return MoECase(f"gpt_oss_20b_decode_t{T}", layer, x, BF16)


def bf16_20b(T: int, seed: int = 0) -> MoECase:
    """The 20b layer of decode_20b (same generator and seed) with T bf16
    tokens ~N(0, 1): the routed/dense crossover sweep over T."""
    assert T >= 1
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, 32, 2880, 2880, 4, BF16, 120, 126, 0.01, 0.02, 0.01)
    x = _real(rng, (T, 2880), 1.0, BF16)
    return MoECase(f"gpt_oss_20b_bf16_t{T}", layer, x, BF16)


def prefill_120b(T: int = 4096, seed: int = 0) -> MoECase:
    """gpt-oss-120b-shaped prefill: E=128, top-4, H=I=2880, T=4096, bf16.

    Expert load is skewed by a per-expert router bias ~N(0, 0.5)."""
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, 128, 2880, 2880, 4, BF16, 120, 126, 0.01, 0.02, 0.5)
    x = _real(rng, (T, 2880), 1.0, BF16)
    return MoECase(f"gpt_oss_120b_prefill_t{T}", layer, x, BF16)


def fp8_20b(T: int = 2048, seed: int = 0, calib_seed: int = 1, calib_tokens: int = 256) -> MoECase:
    """W-MXFP4 A-FP8: the 20b shape with T=2048 and a 256-token calibration
    batch ~N(0, 1) drawn from its own generator."""
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, 32, 2880, 2880, 4, BF16, 120, 126, 0.01, 0.02, 0.01)
    x = _real(rng, (T, 2880), 1.0, BF16)
    crng = np.random.default_rng(calib_seed)
    xc = _real(crng, (calib_tokens, 2880), 1.0, BF16)
    return MoECase(f"gpt_oss_20b_w_mxfp4_a_fp8_t{T}", layer, x, BF16, fp8=True, x_calib=xc)


def small_case(
    seed: int,
    E: int,
    H: int,
    I: int,
    top_k: int,
    T: int,
    act_dtype: str = BF16,
    fp8: bool = False,
    router_bias_std: float = 0.01,
    scale_lo: int = 120,
    scale_hi: int = 126,
) -> MoECase:
    """A layer of arbitrary (small) shape for parity sweeps and edge cases."""
    rng = np.random.default_rng(seed)
    layer = make_layer(rng, E, H, I, top_k, act_dtype, scale_lo, scale_hi, 0.01, 0.1, router_bias_std)
    x = _real(rng, (T, H), 1.0, act_dtype)
    xc = None
    if fp8:
        xc = _real(np.random.default_rng(seed + 1), (64, H), 1.0, act_dtype)
    return MoECase(f"small_s{seed}_e{E}_h{H}_i{I}_k{top_k}_t{T}", layer, x, act_dtype, fp8=fp8, x_calib=xc)


@dataclass
class UnpackCase:
    name: str
    tensors: list  # [(blocks (E, R, K/32, 16) uint8, scales (E, R, K/32) uint8), ...]


def unpack_20b(seed: int = 0, E: int = 32, H: int = 2880, I: int = 2880) -> UnpackCase:
    """Unpack microbench at the 20b expert shapes; nibbles uniform, scales on
    [118, 127].  Draw order: gate_up blocks, gate_up scales, down blocks,
    down scales."""
    rng = np.random.default_rng(seed)
    gub = rng.integers(0, 256, size=(E, 2 * I, H // 32, 16), dtype=np.uint8)
    gus = rng.integers(118, 128, size=(E, 2 * I, H // 32), dtype=np.uint8)
    db = rng.integers(0, 256, size=(E, H, I // 32, 16), dtype=np.uint8)
    ds = rng.integers(118, 128, size=(E, H, I // 32), dtype=np.uint8)
    return UnpackCase(f"unpack_20b_e{E}", [(gub, gus), (db, ds)])


@dataclass
class LinearCase:
    name: str
    x: np.ndarray        # (T, K) in act_dtype storage
    blocks: np.ndarray   # (N, K/32, 16) uint8
    scales: np.ndarray   # (N, K/32) uint8
    bias: Optional[np.ndarray]  # (N,) in act_dtype storage
    act_dtype: str


def linear_case(seed: int, T: int, K: int, N: int, act_dtype: str = BF16, bias: bool = True,
                scale_lo: int = 120, scale_hi: int = 126) -> LinearCase:
    """A weight-only MXFP4 dense layer and its input.  Draw order: blocks,
    scales, bias, x; distributions as the expert weights (nibbles uniform,
    scales on [lo, hi]), bias N(0, 0.01), x N(0, 1)."""
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    blocks = rng.integers(0, 256, size=(N, K // 32, 16), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, size=(N, K // 32), dtype=np.uint8)
    b = _real(rng, (N,), 0.01, act_dtype) if bias else None
    x = _real(rng, (T, K), 1.0, act_dtype)
    return LinearCase(f"linear_s{seed}_t{T}_k{K}_n{N}_{act_dtype}", x, blocks, scales, b, act_dtype)


@dataclass
class Fp8LinearCase:
    name: str
    x: np.ndarray        # (T, K) bf16 bits
    w_codes: np.ndarray  # (N, K) uint8 float8_e4m3fn codes
    w_scale: float       # static per-tensor weight scale
    x_scale: float       # static per-tensor input scale
    bias: Optional[np.ndarray]  # (N,) bf16 bits


def fp8_linear_case(seed: int, T: int, K: int, N: int, bias: bool = True, w_scale: float = 2.0**-8,
                    x_scale: float = 2.0**-6) -> Fp8LinearCase:
    """A dense FP8 E4M3 layer with static per-tensor scales and its input.
    Draw order: codes, bias, x.  Codes uniform over the finite e4m3 codes
    (the two NaN codes are redrawn as zero); bias N(0, 0.01); x N(0, 1).
    The scales are fixed constants, as a calibration would have left them:
    x_scale = 2^-6 puts inputs up to 7 inside the e4m3 range."""
    assert K % 32 == 0 and N % 32 == 0
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    b = _real(rng, (N,), 0.01, BF16) if bias else None
    x = _real(rng, (T, K), 1.0, BF16)
    return Fp8LinearCase(f"fp8_linear_s{seed}_t{T}_k{K}_n{N}", x, codes, w_scale, x_scale, b)


@dataclass
class Int8MoELayer:
    """One INT8 W8A8 MoE layer's parameters (host copies): int8 codes with
    fp32 per-row scales, bf16 bits for the biases and the router."""

    E: int
    H: int
    I: int
    top_k: int
    gate_up_codes: np.ndarray  # (E, 2I, H) int8, rows gate/up interleaved
    gate_up_scale: np.ndarray  # (E, 2I) float32
    gate_up_bias: np.ndarray   # (E, 2I) bf16 bits
    down_codes: np.ndarray     # (E, H, I) int8
    down_scale: np.ndarray     # (E, H) float32
    down_bias: np.ndarray      # (E, H) bf16 bits
    router_w: np.ndarray       # (E, H) bf16 bits
    router_b: np.ndarray       # (E,) bf16 bits


def int8_layer(rng: np.random.Generator, E: int, H: int, I: int, top_k: int, scale_lo: float = 2e-4,
               scale_hi: float = 8e-4, bias_std: float = 0.01, router_std: float = 0.02,
               router_bias_std: float = 0.01) -> Int8MoELayer:
    """Draw order: gate_up codes, scales, bias; down codes, scales, bias;
    router weight, bias.  Codes uniform on [-127, 127]; per-row scales
    uniform on [scale_lo, scale_hi] (fp32), which keeps G of order one at
    H = 2880 with x ~ N(0, 1)."""
    assert H % 32 == 0 and I % 32 == 0
    gu = rng.integers(-127, 128, size=(E, 2 * I, H), dtype=np.int64).astype(np.int8)
    gus = rng.uniform(scale_lo, scale_hi, size=(E, 2 * I)).astype(np.float32)
    gub = _real(rng, (E, 2 * I), bias_std, BF16)
    dn = rng.integers(-127, 128, size=(E, H, I), dtype=np.int64).astype(np.int8)
    dns = rng.uniform(scale_lo, scale_hi, size=(E, H)).astype(np.float32)
    dnb = _real(rng, (E, H), bias_std, BF16)
    rw = _real(rng, (E, H), router_std, BF16)
    rb = _real(rng, (E,), router_bias_std, BF16)
    return Int8MoELayer(E, H, I, top_k, gu, gus, gub, dn, dns, dnb, rw, rb)


@dataclass
class Int8Case:
    name: str
    layer: Int8MoELayer
    x: np.ndarray  # (T, H) bf16 bits

    @property
    def T(self) -> int:
        return self.x.shape[0]


def int8_case(seed: int, E: int, H: int, I: int, top_k: int, T: int, router_bias_std: float = 0.01) -> Int8Case:
    rng = np.random.default_rng(seed)
    layer = int8_layer(rng, E, H, I, top_k, router_bias_std=router_bias_std)
    x = _real(rng, (T, H), 1.0, BF16)
    return Int8Case(f"int8_s{seed}_e{E}_h{H}_i{I}_k{top_k}_t{T}", layer, x)


def int8_20b(T: int, seed: int = 0) -> Int8Case:
    """The gpt-oss-20b shape (E=32, top-4, H=I=2880) as an INT8 W8A8 layer
    with T bf16 tokens ~N(0, 1)."""
    rng = np.random.default_rng(seed)
    layer = int8_layer(rng, 32, 2880, 2880, 4)
    x = _real(rng, (T, 2880), 1.0, BF16)
    return Int8Case(f"gpt_oss_20b_int8_w8a8_t{T}", layer, x)


def int8_layer_to_torch(layer: Int8MoELayer, device):
    """The layer's arrays as device tensors, weights tiled by the library."""
    from mxfp4_quantized_moe_amd import MoEInt8Weights

    return MoEInt8Weights.from_codes(_t(layer.gate_up_codes, device), _t(layer.gate_up_scale, device),
                                     _t(layer.gate_up_bias, device), _t(layer.down_codes, device),
                                     _t(layer.down_scale, device), _t(layer.down_bias, device),
                                     _t(layer.router_w, device), _t(layer.router_b, device), layer.top_k)


def random_weights(seed: int, rows: int, k: int, std: float = 1.0, dtype: str = F32) -> np.ndarray:
    """A dense weight matrix to be packed (pack parity cases)."""
    rng = np.random.default_rng(seed)
    return _real(rng, (rows, k), std, dtype)


# ---------------------------------------------------------------------------
# Device upload (bit-for-bit copies, no arithmetic).
# ---------------------------------------------------------------------------


def _t(a: np.ndarray, device):
    import torch

    if a.dtype == np.uint16:  # raw bf16 bits
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def layer_to_torch(layer: MoELayer, device):
    """The layer's arrays as device tensors, in the binding's MoEWeights."""
    from mxfp4_quantized_moe_amd import MoEWeights

    return MoEWeights(
        gate_up_blocks=_t(layer.gate_up_blocks, device),
        gate_up_scales=_t(layer.gate_up_scales, device),
        gate_up_bias=_t(layer.gate_up_bias, device),
        down_blocks=_t(layer.down_blocks, device),
        down_scales=_t(layer.down_scales, device),
        down_bias=_t(layer.down_bias, device),
        router_w=_t(layer.router_w, device),
        router_b=_t(layer.router_b, device),
        top_k=layer.top_k,
    )


def array_to_torch(a: np.ndarray, device):
    return _t(a, device)


def torch_to_array(t) -> np.ndarray:
    """Device tensor -> numpy (bf16 as raw uint16 bits)."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()
