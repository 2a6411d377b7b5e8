"""Hand-built layers whose outputs are derived by hand (not a test module).

Each builder returns a workloads.MoECase made of explicit codes and biases;
nothing here evaluates the layer.  The expected values, and how they follow
from the pages' rules, are given next to each builder so the CPU oracle and
the GPU path can both be checked against them.

Shared conventions of the builders: E = 2 experts, top_k = 1, H = I = 32 (one
MXFP4 block per row), every scale byte 127 (2^0), bf16 parameters and
activations (the FP8 activation mode needs bf16).  FP4 nibble 2 is 1.0 and
nibble 0 is +0; element 32b + 2j + n of a row is nibble n of byte j of block
b, so "1.0 at column c" is nibble 2 in the low (c even) or high (c odd) half
of byte c // 2.
"""
from __future__ import annotations

import numpy as np

import workloads as W

H = I = 32
E = 2


def _one_at(row: np.ndarray, col: int) -> None:
    """Put the FP4 code 1.0 at column col of a (1, 16) block row."""
    row[0, col // 2] |= np.uint8(2 << (4 * (col % 2)))


def _layer(gate_up_ones, gate_up_bias, down_ones, down_bias, router_ones, router_bias) -> W.MoELayer:
    """gate_up_ones / down_ones / router_ones: lists of (expert, row, column)
    holding 1.0; every other weight is +0.  Biases: dicts {(expert, row): v}
    (router: {expert: v}), all values exactly representable in bf16."""
    gub = np.zeros((E, 2 * I, 1, 16), np.uint8)
    db = np.zeros((E, H, 1, 16), np.uint8)
    for e, r, c in gate_up_ones:
        _one_at(gub[e, r], c)
    for e, r, c in down_ones:
        _one_at(db[e, r], c)
    gus = np.full((E, 2 * I, 1), 127, np.uint8)
    ds = np.full((E, H, 1), 127, np.uint8)
    gb = np.zeros((E, 2 * I), np.float32)
    for (e, r), v in gate_up_bias.items():
        gb[e, r] = v
    dbias = np.zeros((E, H), np.float32)
    for (e, r), v in down_bias.items():
        dbias[e, r] = v
    rw = np.zeros((E, H), np.float32)
    for e, c in router_ones:
        rw[e, c] = 1.0
    rb = np.zeros((E,), np.float32)
    for e, v in router_bias.items():
        rb[e] = v
    bf = W._to_bf16_bits
    return W.MoELayer(E, H, I, 1, gub, gus, bf(gb), db, ds, bf(dbias), bf(rw), bf(rb), W.BF16)


# ---------------------------------------------------------------------------
# The FP8 activation mode by hand.
#
# Expert 0: gate_0 (row 0) = 1.0 * x_0; up_0 (row 1) = 0; gate_1 (row 2) and
# up_1 (row 3) have zero weights and bias 8; down row 0 = 1.0 * h_0, down row
# 1 = 1.0 * h_1, every down bias 0.  Expert 1: zero weights, zero gate_up
# biases, down bias 5 on every row (so a token sent there outputs 5 in every
# column).  Router: logit_0 = x_0, logit_1 = 1.03125 (bias).
#
# x = [1.0625, 0, ..., 0] (bf16-exact), x_scale = 0.5, h_scale = 1/16.
#
# Router on the unquantised x (the router is not quantised: the
# amd/gpt-oss-20b-MoE-Quant-W-MXFP4-A-FP8-KV-FP8 page, "Quantization
# schemes"): logit_0 = 1.0625 > 1.03125, so expert 0 with weight 1.
# x quantised (FP8 static per-tensor, gpt-oss-120b-mxfp4-fp8attn-v2 page,
# FP8 script): 1.0625 / 0.5 = 2.125 lies halfway between the e4m3 values 2.0
# (mantissa 000) and 2.25 (001); round-half-even gives 2.0, dequantised
# 2.0 * 0.5 = 1.0.  (A router reading that value would see 1.0 < 1.03125 and
# pick expert 1.)
# gate_0 = 1.0, up_0 = 0:  h_0 = (0 + 1) * 1.0 * sigmoid(1.702) = 0.84580.
# gate_1 = 8 -> clamped 7, up_1 = 8 -> clamped 7:  h_1 = 8 * 7 *
#   sigmoid(11.914) = 55.99963.
# h quantised: h_0 / (1/16) = 13.53 -> nearest e4m3 in [8, 16) (spacing 1)
#   is 14 -> 14/16 = 0.875;  h_1 / (1/16) = 895.99 > 448 -> saturates to 448
#   -> 448/16 = 28.
# out = 1 * (h_q W_d^T + b_d) = [0.875, 28, 0, ..., 0], exact in bf16.
#
# What the plausible slips give instead:
#   router on the quantised x         -> expert 1: 5 in every column
#   x not quantised (g = 1.0625)      -> h_0 = 0.91286, 14.61 -> 15 -> 0.9375
#   h not requantised                 -> [0.84580, 55.99963, ...]
#   h code not rescaled by h_scale    -> [14, 448, ...]
#   x code not rescaled by x_scale (g = 2.0) -> h_0 = 1.93566, 30.97 -> 30 (spacing
#                                        2 in [16, 32)) -> 1.875
# ---------------------------------------------------------------------------

FP8_X_SCALE = 0.5
FP8_H_SCALE = 1.0 / 16.0
FP8_EXPECTED = np.array([0.875, 28.0] + [0.0] * (H - 2))


def fp8_by_hand() -> W.MoECase:
    layer = _layer(
        gate_up_ones=[(0, 0, 0)],
        gate_up_bias={(0, 2): 8.0, (0, 3): 8.0},
        down_ones=[(0, 0, 0), (0, 1, 1)],
        down_bias={(1, r): 5.0 for r in range(H)},
        router_ones=[(0, 0)],
        router_bias={1: 1.03125},
    )
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0625
    return W.MoECase("fp8_by_hand", layer, W._to_bf16_bits(x), W.BF16, fp8=True, x_calib=None)


# ---------------------------------------------------------------------------
# FP8 calibration by hand (min/max observer, symmetric, per-tensor: the
# gpt-oss-120b-mxfp4-fp8attn-v2 page's FP8 script).
#
# Expert 0: gate_0 (row 0) = 1.0 * x_0 with bias 0, up_0 bias 0; gate_1 bias
# 8, up_1 bias 3 (zero weights).  Expert 1: gate_0 and up_0 biases 8 (zero
# weights).  Router: logit_0 = x_0, logit_1 = 0.5 (bias).
#
# x_calib = [1.0625, -3, 0, ..., 0]:
#   amax(x) = 3 -> s_x = fp32(3 / 448).  3/448 = (1 + 5/7) * 2^-8 and 5/7 =
#   0.101101101...b, so the 23-bit fraction is 10110110110110110110110
#   followed by 110..., which rounds up: bits 0x3BDB6DB7.
#   Routing: 1.0625 > 0.5 -> expert 0.  Its h: h_0 = 1.0625 *
#   sigmoid(1.808375) = 0.91286 -> bf16 0.9140625 (spacing 2^-8 in [0.5, 1));
#   h_1 = (3 + 1) * 7 * sigmoid(11.914) = 27.99981 -> bf16 28.0 (spacing
#   0.125 in [16, 32)).  amax(h) = 28 -> s_h = 28 / 448 = 0.0625 exactly.
#   Expert 1 (not routed) would give h = 8 * 7 * sigmoid(11.914) -> 56 and
#   s_h = 0.125; the unrounded h would give 27.99981 / 448 != 0.0625.
# ---------------------------------------------------------------------------

CALIB_SX_BITS = 0x3BDB6DB7
CALIB_SH = 0.0625


def calib_by_hand() -> W.MoECase:
    layer = _layer(
        gate_up_ones=[(0, 0, 0)],
        gate_up_bias={(0, 2): 8.0, (0, 3): 3.0, (1, 0): 8.0, (1, 1): 8.0},
        down_ones=[(0, 0, 0), (0, 1, 1)],
        down_bias={},
        router_ones=[(0, 0)],
        router_bias={1: 0.5},
    )
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0625
    x[0, 1] = -3.0
    xb = W._to_bf16_bits(x)
    return W.MoECase("calib_by_hand", layer, xb, W.BF16, fp8=True, x_calib=xb.copy())
