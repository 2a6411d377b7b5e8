"""GPU parity of mxfp4_unpack and mxfp4_pack against the oracle (bit-exact)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import device, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _bits_equal_f64(got_f64: np.ndarray, ref_f64: np.ndarray) -> None:
    nan = np.isnan(ref_f64)
    assert np.array_equal(np.isnan(got_f64), nan)
    assert np.array_equal(got_f64[~nan], ref_f64[~nan])
    assert np.array_equal(np.signbit(got_f64[~nan]), np.signbit(ref_f64[~nan]))


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_unpack_exhaustive_bytes_and_scales(dev, out_dtype):
    import torch
    import mxfp4_quantized_moe_amd as mx

    note(f"unpack exhaustive {out_dtype}")
    blocks = np.broadcast_to(np.arange(256, dtype=np.uint8).reshape(16, 16), (256, 16, 16)).copy()
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = mx.mxfp4_unpack(W.array_to_torch(blocks, dev), W.array_to_torch(scales, dev), dt)
    torch.cuda.synchronize()
    got = W.torch_to_array(out)
    got = O.bf16_from_bits(got) if out_dtype == "bf16" else got.astype(np.float64)
    ref = O.mxfp4_unpack(blocks, scales)
    ref = O.round_bf16(ref) if out_dtype == "bf16" else O.round_f32(ref)  # +-Inf beyond range
    _bits_equal_f64(got, ref)


def test_unpack_ragged_rows(dev):
    import torch
    import mxfp4_quantized_moe_amd as mx

    rng = np.random.default_rng(7)
    for rows, k in [(1, 32), (3, 96), (257, 64), (1000, 2880 * 2 // 2)]:
        note(f"unpack ragged rows={rows} k={k}")
        b = rng.integers(0, 256, size=(rows, k // 32, 16), dtype=np.uint8)
        s = rng.integers(100, 140, size=(rows, k // 32), dtype=np.uint8)
        out = mx.mxfp4_unpack(W.array_to_torch(b, dev), W.array_to_torch(s, dev), torch.bfloat16)
        torch.cuda.synchronize()
        _bits_equal_f64(O.bf16_from_bits(W.torch_to_array(out)), O.mxfp4_unpack(b, s))


def test_unpack_20b_expert_shapes_full_size(dev):
    """The unpack workload at full size (gpt-oss-20b expert tensors, 32
    experts each), in the launch configuration the benchmark times: every
    output bit of both tensors, compared one expert at a time.  Scales lie
    in [118, 127], so every value is finite and exact in bf16 and the raw
    bits of the oracle's values (sign of zero included) are the reference."""
    import torch
    import mxfp4_quantized_moe_amd as mx

    case = W.unpack_20b()
    for ti, (b, s) in enumerate(case.tensors):
        note(f"unpack 20b tensor {ti} shape {b.shape}")
        db, ds = W.array_to_torch(b, dev), W.array_to_torch(s, dev)
        out = mx.mxfp4_unpack(db, ds, torch.bfloat16)
        torch.cuda.synchronize()
        for e in range(b.shape[0]):
            got = W.torch_to_array(out[e])
            assert np.array_equal(got, O.bf16_bits(O.mxfp4_unpack(b[e], s[e]))), (ti, e)
        del out, db, ds
        torch.cuda.empty_cache()


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_pack_matches_oracle(dev, in_dtype):
    import torch
    import mxfp4_quantized_moe_amd as mx

    rng = np.random.default_rng(3)
    rows, k = 300, 320
    w = (rng.normal(size=(rows, k)) * np.exp(rng.normal(size=(rows, 1)) * 3)).astype(np.float32)
    # adversarial rows: exact ties of the FP4 grid, zeros, -0.0, subnormals, huge values
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, -0.25, -0.75, -5.0], np.float32)
    w[0, :] = 0.0
    w[0, 5] = -0.0
    w[1, :32] = np.resize(ties, 32)
    w[1, 0] = 6.0
    w[2, :32] = np.float32(1e-40) * np.arange(32)
    w[3, :32] = np.float32(3e38) * np.linspace(-1, 1, 32)
    w[4, :] = np.resize(ties, k) * np.float32(2.0**-120)
    if in_dtype == "bf16":
        bits = W._to_bf16_bits(w)
        src = W.array_to_torch(bits, dev)
        wv = O.bf16_from_bits(bits)
    else:
        src = W.array_to_torch(w, dev)
        wv = w.astype(np.float64)
    note(f"pack {in_dtype}")
    blocks, scales = mx.mxfp4_pack(src)
    torch.cuda.synchronize()
    rb, rs = O.mxfp4_pack(wv)
    assert np.array_equal(W.torch_to_array(scales), rs)
    assert np.array_equal(W.torch_to_array(blocks), rb)


def test_pack_unpack_roundtrip_20b_gate_up(dev):
    """unpack(pack(unpack(b))) == unpack(b) bit-exactly on a full expert tensor,
    and the bytes are identical on canonical blocks (some |code| in {4, 6})."""
    import torch
    import mxfp4_quantized_moe_amd as mx

    rng = np.random.default_rng(0)
    b = rng.integers(0, 256, size=(4, 5760, 90, 16), dtype=np.uint8)
    s = rng.integers(118, 128, size=(4, 5760, 90), dtype=np.uint8)
    note("pack/unpack roundtrip 4 x 5760 x 2880")
    db, ds = W.array_to_torch(b, dev), W.array_to_torch(s, dev)
    v = mx.mxfp4_unpack(db, ds, torch.bfloat16)
    b2, s2 = mx.mxfp4_pack(v)
    v2 = mx.mxfp4_unpack(b2, s2, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(v.view(torch.int16), v2.view(torch.int16))
    mag = np.stack([b & 7, (b >> 4) & 7], -1).reshape(b.shape[:-1] + (32,))
    canon = (mag >= 6).any(-1)
    hb, hs = W.torch_to_array(b2), W.torch_to_array(s2)
    assert np.array_equal(hb[canon], b[canon]) and np.array_equal(hs[canon], s[canon])
    assert (~canon).sum() > 0  # non-canonical blocks exist and were re-encoded


@pytest.mark.parametrize("mats,rows,nb", [(1, 16, 4), (2, 70, 3), (3, 130, 9), (2, 5760, 90), (4, 2880, 90)])
def test_tile_matches_layout_reference(dev, mats, rows, nb):
    """mxfp4_tile is bit-exact against the tiled order's definition, ragged
    rows and chunks included, and at the 20b gate_up / down shapes."""
    import torch
    import mxfp4_quantized_moe_amd as mx
    from tests import tiled_layout as TL

    note(f"tile mats={mats} rows={rows} nb={nb}")
    rng = np.random.default_rng(mats * 1000 + rows + nb)
    blocks = rng.integers(0, 256, (mats, rows, nb, 16), dtype=np.uint8)
    scales = rng.integers(0, 256, (mats, rows, nb), dtype=np.uint8)
    tb, ts = mx.mxfp4_tile(W.array_to_torch(blocks, dev), W.array_to_torch(scales, dev))
    torch.cuda.synchronize()
    rb, rs = TL.tile(blocks, scales)
    assert np.array_equal(W.torch_to_array(tb), rb)
    assert np.array_equal(W.torch_to_array(ts), rs)
