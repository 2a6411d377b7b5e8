"""Reference of the tiled MXFP4 weight order declared in include/mxmoe.h
(test-side host logic, not part of the library).

For `mats` matrices of (rows, k) values with nb = k/32 blocks per row,
RG = ceil(rows/64) row groups, 4*RG row tiles of 16 rows and
NC = ceil(nb/4) chunks of 4 blocks:
  tiled blocks [mats][4RG][NC][64][16]: slot s = 4r + (b ^ ((r >> 2) & 3))
      of piece (m, t, c) holds block 4c+b of row 16t+r;
  tiled scales [mats][RG][NC][64][4]: byte i of dword l = 16b + r of group
      (m, q, c) is the scale of row 64q+16i+r, block 4c+b;
zero wherever the row or block lies past the matrix.
"""
from __future__ import annotations

import numpy as np


def dims(rows: int, nb: int):
    rg = -(-rows // 64)
    return rg, 4 * rg, -(-nb // 4)


def tile_loops(blocks: np.ndarray, scales: np.ndarray):
    """Entry by entry from the definition (small inputs only)."""
    mats, rows, nb = blocks.shape[:3]
    rg, rt4, nc = dims(rows, nb)
    tb = np.zeros((mats, rt4, nc, 64, 16), np.uint8)
    ts = np.zeros((mats, rg, nc, 64, 4), np.uint8)
    for m in range(mats):
        for t in range(rt4):
            for c in range(nc):
                for r in range(16):
                    for b in range(4):
                        row, blk = 16 * t + r, 4 * c + b
                        if row < rows and blk < nb:
                            tb[m, t, c, 4 * r + (b ^ ((r >> 2) & 3))] = blocks[m, row, blk]
        for q in range(rg):
            for c in range(nc):
                for b in range(4):
                    for r in range(16):
                        for i in range(4):
                            row, blk = 64 * q + 16 * i + r, 4 * c + b
                            if row < rows and blk < nb:
                                ts[m, q, c, 16 * b + r, i] = scales[m, row, blk]
    return tb.reshape(-1), ts.reshape(-1)


def tile(blocks: np.ndarray, scales: np.ndarray):
    """Vectorised: pad to whole tiles, then permute axes."""
    mats, rows, nb = blocks.shape[:3]
    rg, rt4, nc = dims(rows, nb)
    pb = np.zeros((mats, 64 * rg, 4 * nc, 16), np.uint8)
    pb[:, :rows, :nb] = blocks
    ps = np.zeros((mats, 64 * rg, 4 * nc), np.uint8)
    ps[:, :rows, :nb] = scales
    # blocks: (m, t, r, c, b, j) -> (m, t, c, r, b', j) with b' = b ^ ((r >> 2) & 3)
    v = pb.reshape(mats, rt4, 16, nc, 4, 16).transpose(0, 1, 3, 2, 4, 5)
    r = np.arange(16)[:, None]
    src_b = np.arange(4)[None, :] ^ ((r >> 2) & 3)  # block held by slot (r, b')
    v = v[:, :, :, np.arange(16)[:, None], src_b]
    # scales: (m, q, i, r, c, b) -> (m, q, c, b, r, i)
    s = ps.reshape(mats, rg, 4, 16, nc, 4).transpose(0, 1, 4, 5, 3, 2)
    return np.ascontiguousarray(v).reshape(-1), np.ascontiguousarray(s).reshape(-1)


def untile(tb: np.ndarray, ts: np.ndarray, mats: int, rows: int, nb: int):
    """Inverse of the tiling (padding dropped)."""
    rg, rt4, nc = dims(rows, nb)
    v = tb.reshape(mats, rt4, nc, 16, 4, 16)  # (m, t, c, r, slot, j)
    r = np.arange(16)[:, None]
    slot_of_b = np.arange(4)[None, :] ^ ((r >> 2) & 3)  # slot holding block b of row r
    v = v[:, :, :, np.arange(16)[:, None], slot_of_b]  # (m, t, c, r, b, j)
    blocks = v.transpose(0, 1, 3, 2, 4, 5).reshape(mats, 64 * rg, 4 * nc, 16)[:, :rows, :nb]
    s = ts.reshape(mats, rg, nc, 4, 16, 4)  # (m, q, c, b, r, i)
    scales = s.transpose(0, 1, 5, 4, 2, 3).reshape(mats, 64 * rg, 4 * nc)[:, :rows, :nb]
    return np.ascontiguousarray(blocks), np.ascontiguousarray(scales)


# ------------------------------------------------- the tiled FP8 order
#
# (N, K) e4m3 codes -> [4RG][NC][64][32] with RG = ceil(N/64), NC =
# ceil(K/128): lane l = 16g + r of (row tile t, chunk c) holds row 16t + r,
# bytes 128c + 16g .. +16 then 128c + 64 + 16g .. +16; zero past N or K.


def fp8_tile_loops(w: np.ndarray) -> np.ndarray:
    """Byte by byte from the definition (small inputs only)."""
    N, K = w.shape
    rt4, nc = 4 * (-(-N // 64)), -(-K // 128)
    out = np.zeros((rt4, nc, 64, 32), np.uint8)
    for t in range(rt4):
        for c in range(nc):
            for lane in range(64):
                g, r = lane >> 4, lane & 15
                row = 16 * t + r
                for j in range(32):
                    k = 128 * c + 16 * g + (j % 16) + 64 * (j // 16)
                    if row < N and k < K:
                        out[t, c, lane, j] = w[row, k]
    return out


def fp8_tile(w: np.ndarray) -> np.ndarray:
    """Vectorised form of fp8_tile_loops."""
    N, K = w.shape
    rt4, nc = 4 * (-(-N // 64)), -(-K // 128)
    pad = np.zeros((16 * rt4, 128 * nc), np.uint8)
    pad[:N, :K] = w
    # [t][r][c][h][g][16] -> [t][c][g][r][h][16]
    v = pad.reshape(rt4, 16, nc, 2, 4, 16).transpose(0, 2, 4, 1, 3, 5)
    return np.ascontiguousarray(v).reshape(rt4, nc, 64, 32)
