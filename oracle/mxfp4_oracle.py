"""Float64 CPU oracle of the MXFP4 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and
bench.py's CPU-baseline leg may use this module; the HIP library never does.

Sources (the pages this follows, cited by page title and section):

* KerasFormers "mxfp4" page (quantization_mxfp4), intro: MXFP4 stores e2m1
  values two per uint8 with one e8m0 power-of-two scale per 32-value block.
* same page, "Primitives": dequantize maps each nibble through the FP4
  codebook and multiplies by 2^(e8m0 - 127); quantize picks the block
  exponent floor(log2(amax)) - 2 and rounds each value to the nearest FP4
  grid point.
* same page, "As a quantize_model scheme": the contracting dimension must be
  a multiple of 32, else a clear error.
* same page, "As GPT-OSS's native format": gate_up_proj is (E, 2I, H),
  down_proj is (E, H, I), biases stay full precision, decode evaluates only
  the top-k routed experts and gives the same output as the dense path.
* gpt-oss-120b-mxfp4-fp8attn-v2 page, "Model Details" (128 experts, top-4,
  hidden 2880) and the FP8 script's comment (float8_e4m3fn, symmetric,
  per-tensor, static scales from a min/max observer).
* amd/gpt-oss-20b-MoE-Quant-W-MXFP4-A-FP8-KV-FP8 page, "Quantization
  schemes": MX FP4 weights with FP8 symmetric per-tensor activations on the
  MoE MLP linears only; the router is not quantised.
* gpt-oss-15.5b-23E-nf4-GPU page, "Notes": the forward is the upstream
  GptOssExperts one (router -> top-4 -> expert MLP -> weighted sum).

Where the pages are silent the layer's task statement fixes the rest: the
codebook {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}, interleaved gate/up
rows, top-k of the logits then a softmax over those k, and the clamped
SwiGLU  out = (up + 1) * gate * sigmoid(1.702 * gate)  with gate <= 7 and
up in [-7, 7].  Readings of points nobody fixes (nibble order, sign of zero,
tie-breaks, rounding modes) are stated next to the code that takes them.

All arithmetic is float64 except where the method itself names a format:
h is rounded to the activation format before down_proj, FP8 codes are
computed from float32 products, and the final output may be rounded to the
output format.

Pins: every function here is checked in tests/test_oracle.py against values
the pages print, closed forms, library routines (torch CPU casts), brute
force or invariants.  None of the functions is "parity unpinned"; the
conventions listed above (nibble order, interleave, s_h recipe) are pinned
for self-consistency only, since no page prints an example of them.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = [
    "fp4_e2m1_value",
    "FP4_CODE",
    "FP4_MAGNITUDES",
    "e8m0_value",
    "mxfp4_unpack",
    "mxfp4_pack",
    "round_float",
    "round_bf16",
    "round_f32",
    "round_e4m3",
    "e4m3_code",
    "e4m3_decode",
    "bf16_bits",
    "bf16_from_bits",
    "widen",
    "route",
    "permute",
    "swiglu_clamped",
    "moe_forward",
    "moe_forward_dense",
    "fp8_static_scale",
    "fp8_quant_dequant",
    "calibrate_fp8",
    "routing_margin",
    "mxfp4_linear",
    "fp8_linear",
    "int8_quant_rows",
    "moe_forward_int8",
]

# ---------------------------------------------------------------------------
# The FP4 (e2m1) codebook and the e8m0 scale.
# ---------------------------------------------------------------------------


def fp4_e2m1_value(nibble: int) -> float:
    """Value of one e2m1 nibble (KerasFormers "mxfp4" page, intro: e2m1).

    Bit 3 is the sign, bits 2..1 the exponent with bias 1, bit 0 the
    mantissa; exponent 0 is subnormal (0 or 0.5).  Nibble 8 is -0.0."""
    s = (nibble >> 3) & 1
    e = (nibble >> 1) & 3
    m = nibble & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


FP4_CODE = np.array([fp4_e2m1_value(n) for n in range(16)], dtype=np.float64)
FP4_MAGNITUDES = FP4_CODE[:8].copy()  # 0, .5, 1, 1.5, 2, 3, 4, 6


def e8m0_value(s) -> np.ndarray:
    """2^(s - 127) for an e8m0 byte ("Primitives": times 2^(e8m0 - 127)).

    Byte 255 is NaN (the OCP e8m0 NaN code; a reading, no page prints it)."""
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


# ---------------------------------------------------------------------------
# unpack / pack ("Primitives").
# ---------------------------------------------------------------------------


def mxfp4_unpack(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise (..., K/32, 16) uint8 blocks with (..., K/32) e8m0 scales.

    Element 32*b + 2*j + n of a row comes from nibble n of byte j of block b,
    with n = 0 the low nibble (a reading: the pages do not fix the nibble
    order).  Returns float64 (..., K); every value is exact."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if blocks.shape[-1] != 16 or blocks.shape[:-1] != scales.shape:
        raise ValueError("blocks must be (..., nb, 16) and scales (..., nb)")
    lo = FP4_CODE[blocks & 0x0F]
    hi = FP4_CODE[blocks >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(blocks.shape[:-1] + (32,))
    vals = vals * e8m0_value(scales)[..., None]
    return vals.reshape(blocks.shape[:-2] + (blocks.shape[-2] * 32,))


def _nearest_fp4_magnitude_index(a: np.ndarray) -> np.ndarray:
    """Index (0..7) of the FP4 magnitude nearest to a >= 0; a tie goes to the
    even index (round-half-to-even on the code, the IEEE default: a reading,
    "Primitives" says only "nearest").  Magnitudes above 6 saturate to 6."""
    d = np.abs(a[..., None] - FP4_MAGNITUDES)
    dmin = d.min(axis=-1, keepdims=True)
    is_min = d == dmin
    idx = np.arange(8)
    # among the (at most two, adjacent) minimisers prefer the even index
    even_min = is_min & (idx % 2 == 0)
    first_even = np.where(even_min.any(axis=-1), np.argmax(even_min, axis=-1), np.argmax(is_min, axis=-1))
    return first_even


def mxfp4_pack(w: np.ndarray):
    """Quantise (..., K) real values to MXFP4 ("Primitives": quantize).

    Per 32-value block: e = floor(log2(amax)) - 2, taken from the exact binary
    exponent and clamped to [-127, 127] (amax = 0 gives e = -127); the scale
    byte is e + 127; each value w / 2^e goes to the nearest FP4 magnitude
    (ties to even, saturating at 6) with the sign bit of w, so -0.0 and small
    negatives give nibble 8.  K % 32 != 0 raises ValueError ("As a
    quantize_model scheme": a clear error).  NaN/Inf inputs are rejected.

    Returns (blocks (..., K/32, 16) uint8, scales (..., K/32) uint8)."""
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[-1]
    if K % 32 != 0:
        raise ValueError(f"MXFP4 needs the contracting dimension to be a multiple of 32, got {K}")
    if not np.all(np.isfinite(w)):
        raise ValueError("mxfp4_pack: NaN/Inf input")
    wb = w.reshape(w.shape[:-1] + (K // 32, 32))
    amax = np.abs(wb).max(axis=-1)
    _, ex = np.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1)  =>  floor(log2 amax) = ex - 1
    e = np.where(amax > 0, ex - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    v = wb / np.ldexp(1.0, e)[..., None]
    idx = _nearest_fp4_magnitude_index(np.abs(v))
    nib = (idx | (np.signbit(wb).astype(np.int64) << 3)).astype(np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# Rounding to the formats the method names.
# ---------------------------------------------------------------------------


def round_float(x, p: int, emin: int, max_finite: float, saturate: bool) -> np.ndarray:
    """Round float64 values to a binary format with p significant bits and
    minimum normal exponent emin, round-half-to-even (IEEE 754 default),
    gradual underflow.  Results beyond max_finite become +-Inf, or +-max_finite
    when saturate is set.  NaN stays NaN; the sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)
        E = np.maximum(ex - 1, emin)
        q = np.ldexp(1.0, E - (p - 1))
        r = np.rint(a / q) * q
        r = np.where(r > max_finite, max_finite if saturate else np.inf, r)
        r = np.where(np.isinf(a), max_finite if saturate else np.inf, r)
        r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, x)


_BF16_MAX = float((2 - 2.0**-7) * 2.0**127)
_F32_MAX = float((2 - 2.0**-23) * 2.0**127)
_E4M3_MAX = 448.0


def round_bf16(x) -> np.ndarray:
    """bfloat16: 8 significant bits, emin -126, overflow to Inf."""
    return round_float(x, 8, -126, _BF16_MAX, saturate=False)


def round_f32(x) -> np.ndarray:
    """binary32: 24 significant bits, emin -126, overflow to Inf."""
    return round_float(x, 24, -126, _F32_MAX, saturate=False)


def round_e4m3(x) -> np.ndarray:
    """float8_e4m3fn: 4 significant bits, bias 7 (emin -6), no Inf, largest
    finite 448; out-of-range values saturate to +-448 (the FP8 scheme is
    symmetric and static, so overflow saturates: a reading)."""
    return round_float(x, 4, -6, _E4M3_MAX, saturate=True)


def e4m3_code(v) -> np.ndarray:
    """Byte encoding of values already on the e4m3fn grid."""
    v = np.asarray(v, dtype=np.float64)
    s = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    E = ex - 1
    normal = a >= 2.0**-6
    e_field = np.where(normal, E + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, E) - 1.0, a / 2.0**-6) * 8
    m_field = np.rint(mant).astype(np.int64)
    code = (s << 7) | (np.where(a == 0, 0, e_field) << 3) | np.where(a == 0, 0, m_field)
    code = np.where(np.isnan(v), 0x7F | (s << 7), code)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Value of an e4m3fn byte: S.EEEE.MMM, bias 7, E=0 subnormal, S.1111.111 NaN."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0**-6, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_from_bits(bits) -> np.ndarray:
    """Widen raw bfloat16 bits to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """Raw bits of float64 values that are already on the bfloat16 grid."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """A tensor in the layer's storage ('bf16' bits or 'f32') as float64."""
    if dtype == "bf16":
        return bf16_from_bits(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Routing.
# ---------------------------------------------------------------------------


def route(x: np.ndarray, w_r: np.ndarray, b_r: np.ndarray, k: int):
    """Router: logits = x W_r^T + b_r in float64 from the unquantised
    activations (the router is excluded from quantisation on the 120b and
    20b pages), take the top-k logits (ties: lower expert id first), then a
    softmax over those k logits.

    Returns (idx (T, k) int32 in descending-logit order, w (T, k) float64,
    logits (T, E) float64)."""
    logits = x @ w_r.T + b_r
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("top_k must be in [1, E]")
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        idx[t] = order[:k]
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return idx, w, logits


def routing_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the gap between the k-th and (k+1)-th largest logit (inf
    when k = E): a float32 router may pick a different set only where this is
    at rounding-error level."""
    s = -np.sort(-logits, axis=1)
    if k >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def permute(idx: np.ndarray, E: int):
    """Group the T*k routed slots by expert, stably by flat slot id t*k + j.

    Returns counts (E,), offsets (E+1,), sorted_slots (T*k,) (flat slot ids in
    expert order) and slot_pos (T*k,) (row of each flat slot in that order)."""
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_slots = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slots)
    slot_pos[sorted_slots] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_slots, slot_pos


# ---------------------------------------------------------------------------
# Expert MLP pieces.
# ---------------------------------------------------------------------------


def swiglu_clamped(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """gate clamped to <= 7, up clamped to [-7, 7],
    h = (up + 1) * gate * sigmoid(1.702 * gate), with the clamped gate inside
    the sigmoid."""
    g = np.minimum(gate, 7.0)
    u = np.clip(up, -7.0, 7.0)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-1.702 * g))
    return (u + 1.0) * g * sig


def fp8_static_scale(amax: float) -> float:
    """Static per-tensor FP8 scale s = amax / 448 in float32 (min/max observer,
    symmetric: the 120b page's FP8 script comment)."""
    return float(np.float32(amax) / np.float32(448.0))


def fp8_quant_dequant(v: np.ndarray, scale: float):
    """FP8 static quantisation: code = e4m3(fp32(fp32(v) * fp32(1/s))) with
    round-half-to-even and saturation to +-448; 1/s is one float32 division.

    Returns (codes as float64 grid values, dequantised values code * s)."""
    inv = np.float32(1.0) / np.float32(scale)
    prod = (np.asarray(v, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)
    q = round_e4m3(prod)
    return q, q * np.float64(np.float32(scale))


def _round_act(h: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return round_bf16(h)
    if act == "f32":
        return round_f32(h)
    raise ValueError(act)


def moe_forward(
    layer,
    x: np.ndarray,
    act_dtype: str,
    fp8: bool = False,
    x_scale: Optional[float] = None,
    h_scale: Optional[float] = None,
    route_override=None,
    return_parts: bool = False,
):
    """The routed MoE layer (only the top-k experts of each token run).

    layer: a workloads.MoELayer (numpy arrays in bf16 bits or fp32).
    x: (T, H) in act_dtype storage.
    fp8: W-MXFP4 A-FP8 mode; x and h are quantised with the static scales
         x_scale and h_scale before gate_up and before down.
    route_override: optional (idx, w) used instead of the oracle's own routing
         (for tokens whose top-k set is decided by a rounding-level margin).

    Steps: route; group slots by expert; per expert dequantise gate_up,
    G = X W^T + b (float64), h = clamped SwiGLU of (G[:, 0::2], G[:, 1::2]),
    round h to the activation format; Y = h W_d^T + b_d; then
    out_t = sum_j w[t, j] * Y(t, j) in slot order j = 0..k-1.

    Returns out (T, H) float64, unrounded (and the parts if asked)."""
    E, H, I, k = layer.E, layer.H, layer.I, layer.top_k
    xf = widen(x, act_dtype)
    T = xf.shape[0]
    w_r = widen(layer.router_w, layer.param_dtype)
    b_r = widen(layer.router_b, layer.param_dtype)
    b_gu = widen(layer.gate_up_bias, layer.param_dtype)
    b_d = widen(layer.down_bias, layer.param_dtype)
    idx, w, logits = route(xf, w_r, b_r, k)
    if route_override is not None:
        idx = np.asarray(route_override[0], dtype=np.int32)
        w = np.asarray(route_override[1], dtype=np.float64)
    counts, offsets, sorted_slots, slot_pos = permute(idx, E)

    if fp8:
        _, x_in = fp8_quant_dequant(xf, x_scale)
    else:
        x_in = xf

    Y = np.zeros((T * k, H), dtype=np.float64)
    h_all = np.zeros((T * k, I), dtype=np.float64)
    for e in range(E):
        sl = sorted_slots[offsets[e] : offsets[e + 1]]
        if sl.size == 0:
            continue
        tok = sl // k
        Wgu = mxfp4_unpack(layer.gate_up_blocks[e], layer.gate_up_scales[e])  # (2I, H)
        G = x_in[tok] @ Wgu.T + b_gu[e]
        h = swiglu_clamped(G[:, 0::2], G[:, 1::2])
        if fp8:
            _, h = fp8_quant_dequant(h, h_scale)
        else:
            h = _round_act(h, act_dtype)
        h_all[sl] = h
        Wd = mxfp4_unpack(layer.down_blocks[e], layer.down_scales[e])  # (H, I)
        Y[sl] = h @ Wd.T + b_d[e]
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        out += w[:, j : j + 1] * Y[np.arange(T) * k + j]
    if return_parts:
        return out, dict(idx=idx, w=w, logits=logits, counts=counts, offsets=offsets,
                         sorted_slots=sorted_slots, slot_pos=slot_pos, h=h_all, Y=Y)
    return out


def mxfp4_linear(x: np.ndarray, blocks: np.ndarray, scales: np.ndarray, bias, act_dtype: str) -> np.ndarray:
    """A weight-only MXFP4 dense layer (KerasFormers "mxfp4" page, "As a
    quantize_model scheme": a Dense kernel is stored as MXFP4 blocks and
    scales, dequantised on the fly, and must have a contracting dimension
    that is a multiple of 32; the bias keeps full precision as in the
    GPT-OSS experts of the next section).

    y = x W^T + b in float64, W = mxfp4_unpack(blocks, scales) (N, K).
    x: (T, K) in act_dtype storage; bias: (N,) in act_dtype storage or None.
    Returns (T, N) float64, unrounded."""
    xf = widen(x, act_dtype)
    if xf.ndim != 2 or blocks.ndim != 3 or xf.shape[1] != blocks.shape[1] * 32:
        raise ValueError("x (T, K) and blocks (N, K/32, 16) must agree on K")
    W = mxfp4_unpack(blocks, scales)
    y = xf @ W.T
    if bias is not None:
        y = y + widen(bias, act_dtype)
    return y


def fp8_linear(x: np.ndarray, w_codes: np.ndarray, w_scale: float, x_scale: float, bias=None) -> np.ndarray:
    """A dense FP8 E4M3 layer with static per-tensor scales (W8A8): the FP8
    attention projections of the gpt-oss-120b-mxfp4-fp8attn-v2 page ("Model
    Details"; "Quantization Recipe", steps 1 and 2: weights and inputs in
    float8_e4m3fn, symmetric, one static scale per tensor kept as
    weight_scale and input_scale).

    W = e4m3 value of each code * w_scale (N, K); x is quantised with
    fp8_quant_dequant at x_scale (the same rule as the MoE FP8 mode);
    y = x_q W^T + b in float64.
    x: (T, K) bf16 bits; w_codes: (N, K) uint8; bias: (N,) bf16 bits or None.
    Returns (T, N) float64, unrounded."""
    xf = widen(x, "bf16")
    w_codes = np.asarray(w_codes)
    if xf.ndim != 2 or w_codes.ndim != 2 or xf.shape[1] != w_codes.shape[1]:
        raise ValueError("x (T, K) and w_codes (N, K) must agree on K")
    _, xq = fp8_quant_dequant(xf, x_scale)
    W = e4m3_decode(w_codes) * np.float64(np.float32(w_scale))
    y = xq @ W.T
    if bias is not None:
        y = y + widen(bias, "bf16")
    return y


def int8_quant_rows(v: np.ndarray):
    """Symmetric int8 with one dynamic scale per row (per token), the W8A8
    scheme of the gpt-oss-20b-BF16-w8a8-llmcompressor page ("Quantization":
    activations int8, symmetric, per-token dynamic).  The scale and the code
    are decided in float32, as a device would: s = fp32(amax|row|) / 127,
    code = clamp(rne(fp32(v) / s), -127, 127); an all-zero row has s = 0 and
    codes 0.  Returns (codes int64 (rows, K), scales float64 (rows,))."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(f), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((f / safe[:, None]).astype(np.float32)).astype(np.float64)
    q = np.clip(q, -127, 127)
    q = np.where(s[:, None] > 0, q, 0.0)
    return q.astype(np.int64), s.astype(np.float64)


def _exact_int_matmul(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """a (n, K) int codes times w (R, K) int8 codes transposed, exactly.

    Every product and every partial sum is an integer of magnitude at most
    127 * 127 * K < 2^53 (K < 2^39), so a float64 matrix product holds them
    all exactly whatever its summation order: the result equals the integer
    product (a float64 product rather than an int64 one only for speed)."""
    K = a.shape[1]
    assert K < 2**39 and np.abs(a).max(initial=0) <= 127
    return a.astype(np.float64) @ w.astype(np.float64).T


def moe_forward_int8(layer8, x: np.ndarray, route_override=None, return_parts: bool = False):
    """The INT8 W8A8 MoE layer (gpt-oss-20b-BF16-w8a8-llmcompressor page,
    "Quantization": weights int8 per output channel with static scales,
    activations int8 per token with dynamic scales, router and biases kept
    in bf16).

    layer8: a workloads.Int8MoELayer (int8 codes, fp32 per-row scales, bf16
    bits elsewhere); x: (T, H) bf16 bits.  Steps: route (as moe_forward);
    x -> int8 per token; per expert G = (x_code W_code^T) s_x s_w + b_gu
    (the integer sums exact); h = clamped SwiGLU, rounded to bf16; h -> int8
    per routed row; Y = (h_code W_code^T) s_h s_w + b_d; out_t =
    sum_j w[t, j] Y(t, j) in slot order.
    Returns out (T, H) float64, unrounded (and the parts if asked)."""
    L = layer8
    E, H, I, k = L.E, L.H, L.I, L.top_k
    xf = bf16_from_bits(x)
    T = xf.shape[0]
    idx, w, _ = route(xf, bf16_from_bits(L.router_w), bf16_from_bits(L.router_b), k)
    if route_override is not None:
        idx = np.asarray(route_override[0], dtype=np.int32)
        w = np.asarray(route_override[1], dtype=np.float64)
    counts, offsets, sorted_slots, slot_pos = permute(idx, E)
    xq, sx = int8_quant_rows(xf)
    b_gu = bf16_from_bits(L.gate_up_bias)
    b_d = bf16_from_bits(L.down_bias)
    Y = np.zeros((T * k, H))
    hb = np.zeros((T * k, I))
    for e in range(E):
        sl = sorted_slots[offsets[e] : offsets[e + 1]]
        if sl.size == 0:
            continue
        tok = sl // k
        acc = _exact_int_matmul(xq[tok], L.gate_up_codes[e])
        G = acc * sx[tok][:, None] * L.gate_up_scale[e].astype(np.float64) + b_gu[e]
        h = round_bf16(swiglu_clamped(G[:, 0::2], G[:, 1::2]))
        hb[sl] = h
        hq, sh = int8_quant_rows(h)
        acc2 = _exact_int_matmul(hq, L.down_codes[e])
        Y[sl] = acc2 * sh[:, None] * L.down_scale[e].astype(np.float64) + b_d[e]
    out = np.zeros((T, H))
    for j in range(k):
        out += w[:, j : j + 1] * Y[np.arange(T) * k + j]
    if return_parts:
        return out, dict(idx=idx, w=w, h=hb, Y=Y, xq=xq, sx=sx)
    return out


def moe_forward_dense(layer, x: np.ndarray, act_dtype: str) -> np.ndarray:
    """Brute force: evaluate every expert for every token and weight by a
    (T, E) score matrix that is zero outside each token's top-k ("As GPT-OSS's
    native format": the dense all-experts path gives identical output).
    Sums over experts in ascending id.  Tiny inputs only."""
    E, k = layer.E, layer.top_k
    xf = widen(x, act_dtype)
    T = xf.shape[0]
    w_r = widen(layer.router_w, layer.param_dtype)
    b_r = widen(layer.router_b, layer.param_dtype)
    b_gu = widen(layer.gate_up_bias, layer.param_dtype)
    b_d = widen(layer.down_bias, layer.param_dtype)
    idx, w, _ = route(xf, w_r, b_r, k)
    score = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            score[t, idx[t, j]] = w[t, j]
    out = np.zeros((T, layer.H))
    for e in range(E):
        Wgu = mxfp4_unpack(layer.gate_up_blocks[e], layer.gate_up_scales[e])
        G = xf @ Wgu.T + b_gu[e]
        h = _round_act(swiglu_clamped(G[:, 0::2], G[:, 1::2]), act_dtype)
        Wd = mxfp4_unpack(layer.down_blocks[e], layer.down_scales[e])
        out += score[:, e : e + 1] * (h @ Wd.T + b_d[e])
    return out


def calibrate_fp8(layer, x_calib: np.ndarray, act_dtype: str):
    """Static FP8 scales from a calibration batch: s_x = amax(x)/448 and
    s_h = amax(h)/448, with h the SwiGLU output of the unquantised
    (activation-format) path over every routed (token, expert) pair, rounded
    to the activation format as it would be stored.  One scale per tensor
    for all experts (the A-FP8 scheme is per-tensor)."""
    xf = widen(x_calib, act_dtype)
    s_x = fp8_static_scale(float(np.abs(xf).max()))
    _, parts = moe_forward(layer, x_calib, act_dtype, return_parts=True)
    s_h = fp8_static_scale(float(np.abs(parts["h"]).max()))
    return s_x, s_h
