"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
values the pages print (tests/golden/), closed forms computed in integers,
library routines (torch CPU casts and ops), brute force on tiny inputs, or
invariants.  A plausible slip anywhere in the oracle (a dropped term, a
wrong sign, swapped nibbles or gate/up rows, a transposed operand) fails at
least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- codebook


def test_codebook_matches_printed_magnitudes():
    printed = [float(r[0]) for r in _read_golden("fp4_codebook.txt")]
    assert list(O.FP4_MAGNITUDES) == printed
    # nibbles 8..15 are the negatives, nibble 8 is negative zero
    for n in range(8):
        assert O.FP4_CODE[n + 8] == -O.FP4_CODE[n]
        assert not math.copysign(1.0, O.FP4_CODE[n])  < 0
        assert math.copysign(1.0, O.FP4_CODE[n + 8]) < 0


def test_codebook_is_e2m1_bit_layout():
    # e2m1: bit3 sign, bits 2..1 exponent (bias 1), bit0 mantissa.  Each
    # magnitude must be representable with 2 exponent bits and 1 mantissa
    # bit, and codes must increase with the unsigned 3-bit field.
    mags = O.FP4_MAGNITUDES
    assert np.all(np.diff(mags) > 0)
    for n in range(1, 8):
        f = Fraction(mags[n]).limit_denominator(4)
        # normal numbers have the form (1 + m/2) * 2^(e-1) for e in 1..3
        e, m = n >> 1, n & 1
        if e:
            assert f == Fraction(2 + m, 2) * Fraction(2) ** (e - 1)
        else:
            assert f == Fraction(1, 2)


# ------------------------------------------------------------------ e8m0


def test_e8m0_matches_torch():
    s = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = O.e8m0_value(np.arange(256))
    assert np.array_equal(mine[:255], s[:255])
    assert np.isnan(mine[255]) and np.isnan(s[255])


# ---------------------------------------------------------------- unpack


def _closed_form_pair(byte, scale):
    """Two values of one byte, from integers: |code| * 2 is an integer in
    {0,1,2,3,4,6,8,12} read off the printed magnitudes."""
    twice = [int(2 * float(r[0])) for r in _read_golden("fp4_codebook.txt")]
    out = []
    for nib in (byte & 0xF, byte >> 4):
        mag = Fraction(twice[nib & 7], 2) * Fraction(2) ** (scale - 127)
        v = float(mag)
        out.append(-v if nib & 8 else v)
    return out


def test_unpack_exhaustive_bytes_and_scales():
    bytes_ = np.arange(256, dtype=np.uint8)
    blocks = np.zeros((256, 16, 16), dtype=np.uint8)  # (scale, block, byte)
    # every block holds all 256 byte values once across 16 blocks x 16 bytes
    blocks[:] = bytes_.reshape(16, 16)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    vals = O.mxfp4_unpack(blocks, scales)  # (256, 512)
    for s in range(255):
        for b in range(256):
            blk, j = divmod(b, 16)
            want = _closed_form_pair(b, s)
            got = vals[s, blk * 32 + 2 * j : blk * 32 + 2 * j + 2]
            assert got[0] == want[0] and got[1] == want[1]
            assert math.copysign(1, got[0]) == math.copysign(1, want[0])
            assert math.copysign(1, got[1]) == math.copysign(1, want[1])
    assert np.all(np.isnan(vals[255]))


def test_unpack_element_order():
    # one nonzero nibble at a time: element 32*b + 2*j + n is nibble n of byte j
    blocks = np.zeros((1, 3, 16), dtype=np.uint8)
    scales = np.full((1, 3), 127, dtype=np.uint8)
    blocks[0, 2, 5] = 0x70  # high nibble of byte 5 of block 2 = code 7 (6.0)
    v = O.mxfp4_unpack(blocks, scales)[0]
    nz = np.nonzero(v)[0]
    assert list(nz) == [2 * 32 + 2 * 5 + 1] and v[nz[0]] == 6.0


def test_unpack_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.mxfp4_unpack(np.zeros((2, 15), np.uint8), np.zeros((2,), np.uint8))


# ------------------------------------------------------------------ pack


def test_pack_rejects_k_not_multiple_of_32():
    with pytest.raises(ValueError):
        O.mxfp4_pack(np.ones((2, 48)))


def test_pack_tie_table():
    rows = _read_golden("pack_ties.txt")
    for inp, exp in rows:
        inp, exp = float(inp), float(exp)
        for sign in (1.0, -1.0):
            w = np.zeros((1, 32))
            # a 6.0 in the block fixes the exponent to 0 (floor(log2 6) - 2);
            # inputs in (6, 8) fix it to 0 by themselves
            w[0, 0] = 6.0 if inp <= 6 else 0.0
            w[0, 1] = sign * inp
            blocks, scales = O.mxfp4_pack(w)
            assert scales[0, 0] == 127
            got = O.mxfp4_unpack(blocks, scales)[0, 1]
            assert got == sign * exp, (inp, sign, got)
            assert math.copysign(1.0, got) == sign


def test_pack_brute_force_nearest():
    rng = np.random.default_rng(3)
    w = rng.normal(size=(64, 64)) * np.exp(rng.normal(size=(64, 1)))
    blocks, scales = O.mxfp4_pack(w)
    deq = O.mxfp4_unpack(blocks, scales)
    wb = w.reshape(64, 2, 32)
    for r in range(64):
        for b in range(2):
            e = int(scales[r, b]) - 127
            amax = np.abs(wb[r, b]).max()
            # scale rule: 2^(e+2) <= amax < 2^(e+3), from the exact exponent
            assert 2.0 ** (e + 2) <= amax < 2.0 ** (e + 3)
            for i in range(32):
                v = wb[r, b, i] / 2.0**e
                # brute force over all 16 signed codes
                cands = [O.fp4_e2m1_value(n) for n in range(16)]
                d = [abs(v - c) for c in cands]
                best = min(d)
                ok = [c for c, dd in zip(cands, d) if dd == best]
                got = deq[r, b * 32 + i] / 2.0**e
                assert got in ok or (abs(v) > 6 and abs(got) == 6)


def test_pack_scale_rule_adversarial():
    for k in range(-120, 120, 7):
        for c in (1.0, 1.5, 6.0 / 4, 7.99 / 4, 1.999999):
            amax = c * 2.0**k  # c in [1, 2) so floor(log2 amax) = k
            w = np.zeros((1, 32))
            w[0, 3] = amax
            _, sc = O.mxfp4_pack(w)
            assert int(sc[0, 0]) - 127 == max(min(k - 2, 127), -127)
    # all-zero block -> scale byte 0, nibbles 0 (or 8 for -0.0)
    w = np.zeros((1, 32))
    w[0, 1] = -0.0
    b, s = O.mxfp4_pack(w)
    assert s[0, 0] == 0 and b[0, 0, 0] == 0x80 and np.all(b[0, 0, 1:] == 0)


def test_pack_roundtrip_on_lattice():
    # "Primitives": quantize is a value-exact inverse on the lattice.
    rng = np.random.default_rng(0)
    blocks = rng.integers(0, 256, size=(40, 8, 16), dtype=np.uint8)
    scales = rng.integers(1, 250, size=(40, 8), dtype=np.uint8)
    v = O.mxfp4_unpack(blocks, scales)
    b2, s2 = O.mxfp4_pack(v)
    v2 = O.mxfp4_unpack(b2, s2)
    assert np.array_equal(v, v2)
    assert np.array_equal(np.signbit(v), np.signbit(v2))
    # bytes are identical on canonical blocks (some |nibble| in {4, 6})
    mag = np.stack([blocks & 7, (blocks >> 4) & 7], -1).reshape(40, 8, 32)
    canon = (mag >= 6).any(axis=-1)
    assert canon.mean() > 0.99
    assert np.array_equal(b2[canon], blocks[canon]) and np.array_equal(s2[canon], scales[canon])


def test_pack_cosine_sanity():
    # Soft check near the page's "~0.98 cosine" for 4-bit RTN on Gaussian weights.
    rng = np.random.default_rng(1)
    w = rng.normal(size=(256, 256))
    v = O.mxfp4_unpack(*O.mxfp4_pack(w))
    cos = (w * v).sum() / np.linalg.norm(w) / np.linalg.norm(v)
    assert 0.97 < cos < 0.999


# ------------------------------------------------------- rounding formats


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(size=20000).astype(np.float32),
        (rng.normal(size=2000) * 1e-39).astype(np.float32),  # subnormal range
        np.float32([3.4e38, -3.39e38, 0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8]),
    ])
    # exact midpoints between neighbouring bf16 values
    base = O.bf16_from_bits(rng.integers(0, 0x7F00, size=5000).astype(np.uint16))
    x = np.concatenate([x, (base * (1 + 2.0**-8)).astype(np.float32)])
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    mine = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(mine, t)
    assert np.array_equal(np.signbit(mine), np.signbit(t))


def test_round_e4m3_matches_torch_and_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3_decode(codes)
    nan = np.isnan(tv)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], tv[~nan])
    grid = np.unique(np.abs(tv[~nan]))
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([mids, -mids, grid, rng.normal(size=5000) * 100, rng.normal(size=500) * 1e-3,
                        [448.0, 449.0, 463.9, 464.0, 465.0, 1e6, -1e6]]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.round_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # the byte encoding inverts the decode on the grid
    assert np.array_equal(O.e4m3_decode(O.e4m3_code(grid)), grid)


def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(2)
    x = rng.normal(size=10000) * np.exp(rng.normal(size=10000) * 20)
    assert np.array_equal(O.round_f32(x), x.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------- routing


def test_route_ties_and_softmax():
    # logits = x when W_r = I and b = 0
    x = np.array([[1.0, 3.0, 2.0, 3.0], [0.0, 0.0, 0.0, 0.0], [-1.0, 5.0, 4.0, 0.0]])
    idx, w, _ = O.route(x, np.eye(4), np.zeros(4), 2)
    assert idx.tolist() == [[1, 3], [0, 1], [1, 2]]
    assert np.allclose(w[0], [0.5, 0.5]) and np.allclose(w[1], [0.5, 0.5])
    # closed form for k = 2: w0 = 1 / (1 + exp(l1 - l0))
    assert abs(w[2, 0] - 1 / (1 + math.exp(4 - 5))) < 1e-15
    idx1, w1, _ = O.route(x, np.eye(4), np.zeros(4), 1)
    assert np.all(w1 == 1.0) and idx1[:, 0].tolist() == [1, 0, 1]


def test_route_brute_force_random():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(50, 16))
    wr = rng.normal(size=(8, 16))
    br = rng.normal(size=8)
    for k in (1, 2, 4, 8):
        idx, w, logits = O.route(x, wr, br, k)
        ref = torch.topk(torch.from_numpy(x @ wr.T + br), k, dim=1)
        assert np.array_equal(idx, ref.indices.numpy())
        sw = torch.softmax(ref.values, dim=1).numpy()
        assert np.allclose(w, sw, rtol=1e-14, atol=0)
        assert np.allclose(w.sum(1), 1.0) and np.all(np.diff(w, axis=1) <= 0)


def test_routing_margin_by_hand():
    """The gap between the k-th and (k+1)-th largest logit, worked by hand;
    zero at a tie that straddles the cut, inf when every expert is chosen."""
    logits = np.array([[0.5, 3.0, -1.0, 2.0], [1.0, 1.0, 1.0, 0.0], [4.0, -2.0, 0.0, 4.0]])
    assert O.routing_margin(logits, 1).tolist() == [1.0, 0.0, 0.0]
    assert O.routing_margin(logits, 2).tolist() == [1.5, 0.0, 4.0]
    assert O.routing_margin(logits, 3).tolist() == [1.5, 1.0, 2.0]
    assert np.all(np.isinf(O.routing_margin(logits, 4)))


def test_permute_invariants_and_brute_force():
    rng = np.random.default_rng(9)
    E, T, k = 7, 33, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, slots, pos = O.permute(idx, E)
    # brute force stable bucket sort
    buckets = [[] for _ in range(E)]
    for s, e in enumerate(idx.ravel()):
        buckets[e].append(s)
    assert slots.tolist() == [s for b in buckets for s in b]
    assert counts.tolist() == [len(b) for b in buckets]
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.sort(slots), np.arange(T * k))
    assert np.array_equal(slots[pos], np.arange(T * k))
    for e in range(E):
        assert np.all(idx.ravel()[slots[offsets[e]:offsets[e + 1]]] == e)


# ----------------------------------------------------------------- SwiGLU


def test_swiglu_special_cases_and_library():
    assert O.swiglu_clamped(np.array([3.0]), np.array([-1.0]))[0] == 0.0
    assert O.swiglu_clamped(np.array([0.0]), np.array([2.0]))[0] == 0.0
    assert O.swiglu_clamped(np.array([100.0]), np.array([0.5]))[0] == O.swiglu_clamped(np.array([7.0]), np.array([0.5]))[0]
    assert O.swiglu_clamped(np.array([1.0]), np.array([100.0]))[0] == O.swiglu_clamped(np.array([1.0]), np.array([7.0]))[0]
    assert O.swiglu_clamped(np.array([1.0]), np.array([-100.0]))[0] == O.swiglu_clamped(np.array([1.0]), np.array([-7.0]))[0]
    assert abs(O.swiglu_clamped(np.array([-1e4]), np.array([1.0]))[0]) < 1e-300
    # below the clamps, (up + 1) * silu(1.702 g) / 1.702 via torch's silu
    rng = np.random.default_rng(0)
    g = rng.uniform(-20, 6.9, size=1000)
    u = rng.uniform(-6.9, 6.9, size=1000)
    ref = (u + 1) * torch.nn.functional.silu(torch.from_numpy(1.702 * g)).numpy() / 1.702
    assert np.allclose(O.swiglu_clamped(g, u), ref, rtol=1e-13, atol=1e-300)


# ---------------------------------------------------- whole layer pins


def test_worked_example_by_hand():
    """E=2, k=1, H=I=32, codes exactly representable, expected by hand.

    Expert 0: gate row 2i is 1.0 at column i, up row 2i+1 is zero; down is
    the identity.  So gate_i = x_i + bg_i, up_i = bu_i and out = h + bd.
    Expert 1 would negate everything; the router sends the token to expert 0
    with weight 1 (softmax over one logit)."""
    H = I = 32
    E = 2
    gub = np.zeros((E, 2 * I, 1, 16), np.uint8)
    db = np.zeros((E, H, 1, 16), np.uint8)
    for i in range(I):
        # 1.0 is nibble 2 (e=1, m=0); -1.0 is nibble 10
        j, n = divmod(i, 2)
        gub[0, 2 * i, 0, j] = 2 << (4 * n)
        gub[1, 2 * i, 0, j] = 10 << (4 * n)
        db[0, i, 0, j] = 2 << (4 * n)
        db[1, i, 0, j] = 10 << (4 * n)
    gus = np.full((E, 2 * I, 1), 127, np.uint8)
    ds = np.full((E, H, 1), 127, np.uint8)
    gubias = np.zeros((E, 2 * I), np.float32)
    gubias[0, 1] = 0.0   # up_0
    gubias[0, 3] = 9.0   # up_1 -> clamped to 7
    gubias[0, 5] = -1.0  # up_2 -> h_2 = 0 whatever the gate
    gubias[0, 6] = 0.5   # gate_3 bias
    gubias[0, 7] = 1.0   # up_3
    dbias = np.zeros((E, H), np.float32)
    dbias[0, 4] = 0.25
    rw = np.zeros((E, H), np.float32)
    rb = np.array([1.0, 0.0], np.float32)
    layer = W.MoELayer(E, H, I, 1, gub, gus, gubias, db, ds, dbias, rw, rb, "f32")
    x = np.zeros((1, H), np.float32)
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 1.0, 8.0, 3.0, -0.5
    out = O.moe_forward(layer, x, "f32")[0]
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    want = np.zeros(H)
    want[0] = (0 + 1) * 1.0 * sig(1.702 * 1.0)
    want[1] = (7 + 1) * 7.0 * sig(1.702 * 7.0)   # gate 8 clamped to 7, up 9 clamped to 7
    want[2] = 0.0                                 # up = -1
    want[3] = (1 + 1) * 0.0 * sig(0.0)            # gate = -0.5 + 0.5 = 0
    want[4] = 0.25                                # bias of down row 4, h_4 = 0
    assert np.allclose(out, O.round_f32(want), rtol=1e-7, atol=0)
    # and the dense brute force agrees
    assert np.allclose(O.moe_forward_dense(layer, x, "f32")[0], out, rtol=1e-12, atol=1e-15)


def _torch_dense_reference(W_gu, b_gu, W_d, b_d, w_r, b_r, x, k):
    """Independent float64 MoE with torch library routines on dense float weights."""
    import torch.nn.functional as F

    x = torch.from_numpy(x)
    logits = F.linear(x, torch.from_numpy(w_r), torch.from_numpy(b_r))
    top = torch.topk(logits, k, dim=1)
    wts = torch.softmax(top.values, dim=1)
    out = torch.zeros(x.shape[0], W_d.shape[1])
    out = out.double()
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(top.indices[t, j])
            G = F.linear(x[t], torch.from_numpy(W_gu[e]), torch.from_numpy(b_gu[e]))
            gate, up = G[0::2].clamp(max=7.0), G[1::2].clamp(-7.0, 7.0)
            h = (up + 1) * gate * torch.sigmoid(1.702 * gate)
            y = F.linear(h, torch.from_numpy(W_d[e]), torch.from_numpy(b_d[e]))
            out[t] += wts[t, j] * y
    return out.numpy()


def test_layer_matches_torch_dense_float_moe_on_grid():
    """Special case: weights on the FP4 grid are exactly their dequantisation,
    so the MXFP4 layer must equal a plain float MoE ("experts expanded to
    float at build", KerasFormers "mxfp4" page, "As GPT-OSS's native
    format") computed with torch library routines."""
    rng = np.random.default_rng(11)
    E, H, I, k, T = 5, 64, 96, 2, 12
    mags = np.array([float(r[0]) for r in _read_golden("fp4_codebook.txt")])
    def grid(shape):
        return mags[rng.integers(0, 8, size=shape)] * rng.choice([-1.0, 1.0], size=shape) * 2.0 ** rng.integers(-3, 2, size=shape[:-1] + (1,))
    W_gu = grid((E, 2 * I, H))
    W_d = grid((E, H, I))
    gub, gus = O.mxfp4_pack(W_gu)
    db, ds = O.mxfp4_pack(W_d)
    b_gu = rng.normal(size=(E, 2 * I)).astype(np.float32)
    b_d = rng.normal(size=(E, H)).astype(np.float32)
    w_r = rng.normal(size=(E, H)).astype(np.float32)
    b_r = rng.normal(size=E).astype(np.float32)
    x = (rng.normal(size=(T, H)) * 0.3).astype(np.float32)
    layer = W.MoELayer(E, H, I, k, gub, gus, b_gu, db, ds, b_d, w_r, b_r, "f32")
    # round h to f32 in the oracle; compare against the unrounded torch path
    ours = O.moe_forward(layer, x, "f32")
    ref = _torch_dense_reference(W_gu, b_gu.astype(np.float64), W_d, b_d.astype(np.float64),
                                 w_r.astype(np.float64), b_r.astype(np.float64), x.astype(np.float64), k)
    assert np.max(np.abs(ours - ref)) <= 1e-6 * np.max(np.abs(ref))


@pytest.mark.parametrize("seed,E,k,act", [(0, 4, 2, "f32"), (1, 6, 3, "bf16"), (2, 3, 3, "bf16"), (3, 8, 1, "f32")])
def test_routed_equals_dense(seed, E, k, act):
    case = W.small_case(seed, E, 64, 32, k, 9, act_dtype=act)
    r = O.moe_forward(case.layer, case.x, act)
    d = O.moe_forward_dense(case.layer, case.x, act)
    assert np.max(np.abs(r - d)) <= 1e-12 * np.max(np.abs(d))


def test_tiny_config_routed_equals_dense():
    case = W.tiny()
    r = O.moe_forward(case.layer, case.x, "f32")
    d = O.moe_forward_dense(case.layer, case.x, "f32")
    assert np.max(np.abs(r - d)) <= 1e-12 * np.max(np.abs(d))


def test_decode_dequant_ratio():
    # "~8x less dequant per layer" for single-token decode: E / k = 32 / 4 on the 20b shape
    case = W.decode_20b(T=1)
    _, parts = O.moe_forward(case.layer, case.x, "bf16", return_parts=True)
    active = int((parts["counts"] > 0).sum())
    assert active == 4 and case.layer.E / active == 8


def test_footprint_closed_form():
    g = {r[0]: r[1:] for r in _read_golden("footprint.txt")}
    L, E, H, I = (int(g[n][0]) for n in ("layers", "experts", "hidden", "intermediate"))
    weights = L * E * (2 * I * H + H * I)
    packed = weights // 2 + weights // 32  # nibbles + one e8m0 byte per 32 values
    gib = packed / 2**30
    gb16 = weights * 2 / 1e9
    assert abs(gib - float(g["packed_gib"][0])) <= float(g["packed_gib"][1]) * float(g["packed_gib"][0])
    assert abs(gb16 - float(g["bf16_gb"][0])) <= float(g["bf16_gb"][1]) * float(g["bf16_gb"][0])
    # the layout the library takes has exactly this many bytes per expert
    lay = W.make_layer(np.random.default_rng(0), 1, H, I, 1, "bf16", 120, 126, 0.01, 0.02, 0.01)
    assert lay.gate_up_blocks.nbytes + lay.gate_up_scales.nbytes + lay.down_blocks.nbytes + lay.down_scales.nbytes == packed // (L * E)


# ------------------------------------------------------------------- FP8


def test_fp8_quant_dequant_and_scale():
    s = O.fp8_static_scale(4.375)
    assert s == float(np.float32(4.375) / np.float32(448))
    v = np.array([0.0, 1.0, -4.375, 10.0, 1e-6])
    q, d = O.fp8_quant_dequant(v, s)
    inv = np.float32(1) / np.float32(s)
    ref = torch.from_numpy(np.clip((v.astype(np.float32) * inv), -448, 448).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(q, ref)
    assert q[3] == 448.0 and abs(q[2]) == 448.0
    assert np.array_equal(d, q * np.float64(np.float32(s)))


def test_fp8_layer_by_hand():
    """The FP8 activation mode on a layer whose output was derived by hand
    (tests/hand_cases.py gives the derivation): router on the unquantised x,
    x quantised with x_scale before gate_up, h requantised with h_scale
    (saturating) before down.  gpt-oss-120b-mxfp4-fp8attn-v2 page, FP8 script
    (float8_e4m3fn, symmetric, per-tensor, static); amd/gpt-oss-20b-MoE-Quant-
    W-MXFP4-A-FP8-KV-FP8 page, "Quantization schemes" (router not quantised,
    activations of the MoE linears FP8 per-tensor)."""
    from tests import hand_cases as HC

    case = HC.fp8_by_hand()
    out, parts = O.moe_forward(case.layer, case.x, "bf16", fp8=True, x_scale=HC.FP8_X_SCALE,
                               h_scale=HC.FP8_H_SCALE, return_parts=True)
    assert parts["idx"][0, 0] == 0  # routed on x, not on its FP8 value
    assert np.array_equal(out[0], HC.FP8_EXPECTED)
    # the bf16 path of the same layer: h_0 = 1.0625 * sigmoid(1.808375) =
    # 0.91286 -> bf16 0.9140625 (spacing 2^-8), h_1 = 55.99963 -> bf16 56
    plain = O.moe_forward(case.layer, case.x, "bf16")[0]
    assert plain[0] == 0.9140625 and plain[1] == 56.0 and not np.any(plain[2:])


def test_fp8_calibration_by_hand():
    """Static scales from a one-token calibration batch, derived by hand
    (tests/hand_cases.py): s_x = amax(x)/448 in fp32 and s_h = amax of the
    bf16 h of the routed expert / 448."""
    from tests import hand_cases as HC

    case = HC.calib_by_hand()
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    assert np.float32(s_x).view(np.uint32) == HC.CALIB_SX_BITS
    assert s_h == HC.CALIB_SH


def test_fp8_mode_error_is_fp8_sized():
    case = W.small_case(4, 4, 64, 64, 2, 16, act_dtype="bf16", fp8=True)
    s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
    ref = O.moe_forward(case.layer, case.x, "bf16")
    q = O.moe_forward(case.layer, case.x, "bf16", fp8=True, x_scale=s_x, h_scale=s_h)
    rel = np.max(np.abs(q - ref)) / np.max(np.abs(ref))
    assert 1e-3 < rel < 0.15  # e4m3 has 3 mantissa bits: a few percent, not zero


# ------------------------------------------------------------ dense MXFP4 linear


def test_linear_exact_integer_closed_form():
    """Grid weights at scale byte 127 (value 1) times small integer inputs:
    every product and sum is an exact multiple of 1/2, so y is the int64
    product of the doubled weights with x, halved, plus an integer bias."""
    rng = np.random.default_rng(7)
    T, K, N = 9, 96, 40
    codes = rng.integers(0, 16, size=(N, K))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], dtype=np.int64)  # 2 x e2m1 value
    nib = codes.reshape(N, K // 32, 16, 2)
    blocks = (nib[..., 0] | (nib[..., 1] << 4)).astype(np.uint8)
    scales = np.full((N, K // 32), 127, dtype=np.uint8)
    x = rng.integers(-8, 9, size=(T, K)).astype(np.float32)
    b = rng.integers(-5, 6, size=N).astype(np.float32)
    y = O.mxfp4_linear(x, blocks, scales, b, "f32")
    exact = (x.astype(np.int64) @ twice[codes].T) / 2.0 + b
    assert np.array_equal(y, exact)
    assert np.array_equal(O.mxfp4_linear(x, blocks, scales, None, "f32"), exact - b)


def test_linear_rejects_mismatched_k():
    blocks = np.zeros((4, 2, 16), dtype=np.uint8)
    scales = np.zeros((4, 2), dtype=np.uint8)
    with pytest.raises(ValueError):
        O.mxfp4_linear(np.zeros((3, 48), np.float32), blocks, scales, None, "f32")


def test_linear_is_the_down_projection_of_the_layer():
    """With one expert, top-1 and the identity router weight of 1, the
    layer's down step is this linear on h: check the linear against the
    layer's own parts (Y = h W_d^T + b_d) on a tiny random layer."""
    case = W.small_case(3, 1, 64, 32, 1, 5, act_dtype="f32")
    out, parts = O.moe_forward(case.layer, case.x, "f32", return_parts=True)
    L = case.layer
    y = O.mxfp4_linear(parts["h"].astype(np.float32), L.down_blocks[0], L.down_scales[0], L.down_bias[0], "f32")
    assert np.allclose(y, parts["Y"], rtol=1e-6, atol=1e-6)
    assert np.allclose(out, parts["Y"])  # top-1 of one expert: weight 1


# ------------------------------------------------------- dense FP8 layer


def _bf16(v):
    return O.bf16_bits(np.asarray(v, dtype=np.float64))


def test_fp8_linear_exact_closed_form():
    """Hand-encoded e4m3 codes (S.EEEE.MMM, bias 7: 0x38 = 1, 0x40 = 2,
    0xBC = -1.5, 0x48 = 4, 0x30 = 0.5) and power-of-two scales; x on the
    grid x_scale * e4m3 so its quantisation is exact: y by hand."""
    w_codes = np.array([[0x38, 0x40, 0xBC, 0x48], [0x30, 0x38, 0x38, 0xC0]], dtype=np.uint8)  # rows of W / w_scale
    w_vals = np.array([[1, 2, -1.5, 4], [0.5, 1, 1, -2]])
    w_scale, x_scale = 0.5, 0.25
    x_grid = np.array([[1, 2, -3, 0.5], [4, -1, 0, 6]])
    x = _bf16(x_grid * x_scale)
    b = _bf16([1.0, -2.0])
    y = O.fp8_linear(x, w_codes, w_scale, x_scale, b)
    expected = np.array([[sum(x_grid[t, k] * x_scale * w_vals[n, k] * w_scale for k in range(4)) + [1.0, -2.0][n]
                          for n in range(2)] for t in range(2)])
    assert np.array_equal(y, expected)
    assert np.array_equal(O.fp8_linear(x, w_codes, w_scale, x_scale, None), expected - np.array([1.0, -2.0]))


def test_fp8_linear_matches_torch_float8():
    """Against torch's own float8_e4m3fn: its decode of the weight codes and
    its round-to-nearest cast of fp32(x) * fp32(1/x_scale) (inputs kept
    inside +-448 x_scale, where no saturation is involved)."""
    rng = np.random.default_rng(5)
    T, K, N = 6, 64, 5
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00  # no NaN codes
    w_scale, x_scale = 0.0123, 0.0071
    x = _bf16(rng.normal(0, 1, size=(T, K)))
    b = _bf16(rng.normal(0, 0.1, size=N))
    y = O.fp8_linear(x, codes, w_scale, x_scale, b)
    wt = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(w_scale))
    xf = torch.from_numpy(O.bf16_from_bits(x).astype(np.float32))
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(x_scale, dtype=torch.float32)
    assert float((xf * inv).abs().max()) < 448
    xq = (xf * inv).to(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(x_scale))
    ref = xq @ wt.T + torch.from_numpy(O.bf16_from_bits(b))
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_fp8_linear_saturates_inputs():
    """x beyond 448 x_scale contributes +-448 x_scale (static scheme,
    saturating cast)."""
    w_codes = np.array([[0x38, 0x38]], dtype=np.uint8)  # W = [1, 1] * w_scale
    x = _bf16([[1000.0, -5000.0]])
    y = O.fp8_linear(x, w_codes, 1.0, 1.0, None)
    assert np.array_equal(y, np.array([[448.0 - 448.0]]))
    y = O.fp8_linear(_bf16([[1000.0, 3.0]]), w_codes, 1.0, 1.0, None)
    assert np.array_equal(y, np.array([[451.0]]))


def test_fp8_linear_rejects_mismatched_k():
    with pytest.raises(ValueError):
        O.fp8_linear(_bf16(np.zeros((2, 32))), np.zeros((3, 64), np.uint8), 1.0, 1.0)


# ------------------------------------------------------ int8 W8A8 layer


def test_int8_quant_rows_matches_torch():
    """Scale fp32(amax) / 127 and code round-half-to-even(fp32 v / s),
    clamped to +-127, against torch's fp32 division and torch.round."""
    rng = np.random.default_rng(11)
    v = O.bf16_from_bits(_bf16(rng.normal(0, 2, size=(7, 96))))
    v[3, 5] = 0.0  # a zero among the values
    q, s = O.int8_quant_rows(v)
    t = torch.from_numpy(v.astype(np.float32))
    ts = t.abs().amax(dim=1) / torch.tensor(127.0, dtype=torch.float32)
    tq = torch.round(t / ts[:, None]).clamp(-127, 127).to(torch.int64)
    assert np.array_equal(s, ts.numpy().astype(np.float64))
    assert np.array_equal(q, tq.numpy())
    # the largest magnitude of a row always maps to +-127
    for r in range(v.shape[0]):
        j = int(np.argmax(np.abs(v[r])))
        assert abs(q[r, j]) == 127


def test_int8_quant_rows_special_cases():
    q, s = O.int8_quant_rows(np.zeros((2, 32)))
    assert np.all(q == 0) and np.all(s == 0)
    row = np.zeros((1, 32))
    row[0, 7] = -3.0
    q, s = O.int8_quant_rows(row)
    assert s[0] == np.float64(np.float32(3.0) / np.float32(127.0))
    assert q[0, 7] == -127 and np.count_nonzero(q) == 1


def test_int8_integer_sums_are_exact():
    """127 * 127 * 2880 < 2^31: the int32 sums of a row are exact, and the
    oracle keeps them as integers (x scale 1 when amax = 127)."""
    L = W.int8_case(2, 1, 2880, 32, 1, 1).layer
    L.gate_up_codes[:] = 127
    x = _bf16(np.full((1, 2880), 127.0))
    out, parts = O.moe_forward_int8(L, x, return_parts=True)
    assert np.array_equal(parts["xq"], np.full((1, 2880), 127))
    assert parts["sx"][0] == 1.0


def test_int8_layer_matches_dense_brute_force():
    """Every expert for every token, weighted by a (T, E) matrix that is
    zero outside the top-k, written out here from the definition with plain
    loops over experts (tiny inputs)."""
    case = W.int8_case(7, 5, 64, 32, 2, 9)
    L = case.layer
    out = O.moe_forward_int8(L, case.x)
    xf = O.bf16_from_bits(case.x)
    idx, w, _ = O.route(xf, O.bf16_from_bits(L.router_w), O.bf16_from_bits(L.router_b), L.top_k)
    xq, sx = O.int8_quant_rows(xf)
    ref = np.zeros_like(out)
    for t in range(case.T):
        for e in range(L.E):
            hit = [j for j in range(L.top_k) if idx[t, j] == e]
            if not hit:
                continue
            G = np.array([sum(int(xq[t, c]) * int(L.gate_up_codes[e, r, c]) for c in range(L.H))
                          for r in range(2 * L.I)], dtype=np.float64)
            G = G * sx[t] * L.gate_up_scale[e].astype(np.float64) + O.bf16_from_bits(L.gate_up_bias[e])
            h = O.round_bf16(O.swiglu_clamped(G[0::2], G[1::2]))[None, :]
            hq, sh = O.int8_quant_rows(h)
            Y = (hq[0] @ L.down_codes[e].astype(np.int64).T) * sh[0] * L.down_scale[e].astype(np.float64)
            ref[t] += w[t, hit[0]] * (Y + O.bf16_from_bits(L.down_bias[e]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
