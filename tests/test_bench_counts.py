"""The benchmark's algorithmic work per launch, against closed forms worked
by hand: the roofline fractions bench.py reports divide by these."""
from types import SimpleNamespace

import bench


def _case(E, k, H, I, T, act="bf16", fp8=False, param="bf16"):
    layer = SimpleNamespace(E=E, top_k=k, H=H, I=I, param_dtype=param)
    return SimpleNamespace(layer=layer, T=T, act_dtype=act, fp8=fp8)


def test_prefill_flops_120b():
    """gate_up: 2 flop x 16384 routed rows x 5760 x 2880; down half of it."""
    c = _case(128, 4, 2880, 2880, 4096)
    assert bench.expert_gemm_flops(c, 0) == 2 * 16384 * 5760 * 2880 == 543_581_798_400
    assert bench.expert_gemm_flops(c, 1) == 2 * 16384 * 2880 * 2880
    # the dense path runs every token through all 128 experts
    assert bench.expert_gemm_flops(c, 0, dense=True) == 32 * bench.expert_gemm_flops(c, 0)


def test_decode_bytes_20b_one_token():
    """One token routed to 4 experts: each expert's gate_up is 5760 rows x 90
    blocks of 17 bytes (16 nibble bytes + 1 scale) plus 5760 bf16 biases;
    then x (2880 bf16) in and h (4 x 2880 bf16) out."""
    c = _case(32, 4, 2880, 2880, 1)
    per_expert = 5760 * 90 * 17 + 5760 * 2
    assert per_expert == 8_824_320
    assert bench.expert_gemm_bytes(c, 0, 4) == 4 * per_expert + 2880 * 2 + 4 * 2880 * 2 == 35_326_080
    # down: 2880 rows x 90 blocks + bias per expert, h in and Y (bf16) out
    assert bench.expert_gemm_bytes(c, 1, 4) == 4 * (2880 * 90 * 17 + 2880 * 2) + 4 * 2880 * 2 + 4 * 2880 * 2


def test_fp8_mode_activation_bytes():
    """FP8 mode: x and h move as one byte per element."""
    c = _case(32, 4, 2880, 2880, 2048, fp8=True)
    w = 5760 * 90 * 17 + 5760 * 2
    assert bench.expert_gemm_bytes(c, 0, 32) == 32 * w + 2048 * 2880 + 2048 * 4 * 2880


def test_decode_step_bytes_20b_one_token():
    """A whole one-token step: the router (32 x 2880 bf16 weights + 32 bf16
    biases), 4 routed experts of 13,236,480 bytes each (both matrices'
    nibbles, scales and biases), x in and out (2880 bf16 each)."""
    c = _case(32, 4, 2880, 2880, 1)
    expert = 5760 * 90 * 17 + 5760 * 2 + 2880 * 90 * 17 + 2880 * 2
    assert expert == 13_236_480
    assert bench.step_bytes(c, 4) == 32 * 2880 * 2 + 32 * 2 + 4 * expert + 2 * 2880 * 2 == 53_141_824

