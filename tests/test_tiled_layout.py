"""The test-side reference of the tiled weight order: the vectorised form
agrees with the entry-by-entry definition, the inverse restores the row
order, and padding is zero."""
import numpy as np
import pytest

from tests import tiled_layout as TL


@pytest.mark.parametrize("mats,rows,nb", [(1, 16, 4), (2, 70, 3), (1, 130, 9), (3, 64, 8), (1, 5, 1)])
def test_vectorised_matches_definition(mats, rows, nb):
    rng = np.random.default_rng(rows * 100 + nb)
    blocks = rng.integers(0, 256, (mats, rows, nb, 16), dtype=np.uint8)
    scales = rng.integers(0, 256, (mats, rows, nb), dtype=np.uint8)
    a = TL.tile_loops(blocks, scales)
    b = TL.tile(blocks, scales)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    rg, rt4, nc = TL.dims(rows, nb)
    assert a[0].size == mats * rt4 * nc * 1024 and a[1].size == mats * rg * nc * 256
    back = TL.untile(b[0], b[1], mats, rows, nb)
    assert np.array_equal(back[0], blocks) and np.array_equal(back[1], scales)
    # every byte lands once; the rest is zero padding
    nz = np.ones_like(blocks)
    pad = TL.tile(nz, np.ones_like(scales))
    assert int(pad[0].sum()) == blocks.size and int(pad[1].sum()) == scales.size


def test_piece_slots_are_a_permutation():
    r = np.arange(16)[:, None]
    b = np.arange(4)[None, :]
    slots = 4 * r + (b ^ ((r >> 2) & 3))
    assert sorted(slots.ravel().tolist()) == list(range(64))
    # lanes r = 0..15 of one lane group (fixed b) touch 16 distinct 16-byte
    # slots whose positions mod 4 cover every bank group equally
    for bb in range(4):
        col = slots[:, bb]
        assert len(set(col.tolist())) == 16
        assert sorted((col % 4).tolist()) == sorted([0, 1, 2, 3] * 4)


@pytest.mark.parametrize("N,K", [(32, 32), (64, 128), (96, 160), (160, 288)])
def test_fp8_tile_vectorised_matches_definition(N, K):
    rng = np.random.default_rng(N + K)
    w = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    assert np.array_equal(TL.fp8_tile(w), TL.fp8_tile_loops(w))


def test_fp8_tile_is_a_permutation_plus_zeros():
    """Every code lands exactly once; the rest of the tiled tensor is zero."""
    N, K = 96, 160
    w = (np.arange(N * K, dtype=np.int64) % 251 + 1).astype(np.uint8).reshape(N, K)  # no zero codes
    t = TL.fp8_tile(w)
    assert np.count_nonzero(t) == N * K
    assert sorted(t[t != 0].tolist()) == sorted(w.ravel().tolist())
