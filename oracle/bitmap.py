"""Oracle bitmap-tile format: encoder, validating decoder and byte count.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the follow-up summary of the pages (gist.science, section "Problematica",
third point): CSR-like position metadata costs as much as the values at about 50%
sparsity, and a bitmap (one bit per position) cuts that metadata at the price of
more decoding work on chip.  The pages give no layout; the readings taken here:

B1  64 x 64 tiles in the Tiled-CSL order (row-block-major, t = bm * ceil(K/64) + bk).
B2  Positions of a tile are numbered in the operand order of the 16x16x32 fp16 MFMA, so
    that each of a wavefront's 64 lanes owns the 64 positions it feeds to the matrix
    unit: lane l (0..63), bit b (0..63) of its mask stands for chunk g = b // 8 and
    element e = b % 8, i.e. tile row 16 * (g // 2) + l % 16 and tile column
    32 * (g % 2) + 8 * (l // 16) + e.  Positions outside the matrix are never set.
B3  A tile with at least one kept entry stores the 64 lane masks (64-bit, little-endian:
    lane l at words 2l (bits 0..31) and 2l + 1 (bits 32..63)), then the kept fp16 bit
    patterns chunk by chunk: for g = 0..7, the values of bits 8g..8g+7 of lanes 0..63, lane
    after lane, each lane's in ascending bit order; padded with 0x0000 to a multiple of 8
    values (whole 16-byte vectors).  Value v sits in the low (v even) or high (v odd) 16
    bits of word 128 + v // 2.  A tile with no kept entry stores nothing; offsets are T+1
    entries in 16-byte units, offsets[0] = 0.
B4  The mask decides what is stored, as in the Tiled-CSL reading R5 (a kept +0 or -0 is
    stored, and -0 survives the round trip).
"""
from __future__ import annotations

import numpy as np

from .tiled_csl import FormatError, grid

TILE = 64
MASK_WORDS = 2 * 64


def position(lane: int, bit: int):
    """(row, column) inside the tile of lane `lane`, mask bit `bit` (B2)."""
    g, e = divmod(bit, 8)
    return 16 * (g // 2) + lane % 16, 32 * (g % 2) + 8 * (lane // 16) + e


def lane_bit(r: int, c: int):
    """Inverse of `position`: (lane, bit) of tile row r, column c."""
    lane = r % 16 + 16 * ((c % 32) // 8)
    g = 2 * (r // 16) + c // 32
    return lane, 8 * g + c % 8


def tile_bytes(n_kept: int) -> int:
    """Bytes of one tile: masks + values rounded up to 8 (B3); 0 for an empty tile."""
    if n_kept == 0:
        return 0
    return 8 * 64 + 16 * ((n_kept + 7) // 8)


def encode(A16: np.ndarray, mask: np.ndarray):
    """Bitmap encoding of (A16, mask): (words uint32[total], offsets uint32[T+1]) per B1-B4."""
    M, K = A16.shape
    MB, KT, _ = grid(M, K, TILE, TILE)
    chunks, offs = [], [0]
    for bm in range(MB):
        for bk in range(KT):
            r0, c0 = bm * TILE, bk * TILE
            sub_m = mask[r0:r0 + TILE, c0:c0 + TILE] != 0
            sub_a = A16[r0:r0 + TILE, c0:c0 + TILE]
            n = int(sub_m.sum())
            if n == 0:
                offs.append(offs[-1])
                continue
            masks = [0] * 64
            for r, c in zip(*np.nonzero(sub_m)):
                lane, bit = lane_bit(int(r), int(c))
                masks[lane] |= 1 << bit
            vals = []
            for g in range(8):                    # chunk by chunk, lane after lane
                for lane in range(64):
                    for bit in range(8 * g, 8 * g + 8):
                        if (masks[lane] >> bit) & 1:
                            r, c = position(lane, bit)
                            vals.append(int(sub_a[r, c]))
            vals += [0] * ((-len(vals)) % 8)
            blob = np.concatenate([np.asarray(masks, dtype=np.uint64).view(np.uint32),
                                   np.asarray(vals, dtype=np.uint16).view(np.uint32)])
            chunks.append(blob)
            offs.append(offs[-1] + blob.size // 4)
    words = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.uint32)
    return words.astype(np.uint32), np.asarray(offs, dtype=np.uint32)


def decode(words: np.ndarray, offsets: np.ndarray, M: int, K: int) -> np.ndarray:
    """Dense fp16 bit patterns of a bitmap encoding; raises FormatError when it is not valid."""
    words = np.asarray(words, dtype=np.uint32)
    offsets = np.asarray(offsets, dtype=np.int64)
    MB, KT, T = grid(M, K, TILE, TILE)
    if offsets.shape != (T + 1,) or offsets[0] != 0 or np.any(np.diff(offsets) < 0):
        raise FormatError("offsets must be non-decreasing from 0 with T+1 entries")
    if 4 * offsets[-1] != words.size:
        raise FormatError("last offset must match the blob size")
    A = np.zeros((M, K), dtype=np.uint16)
    for t in range(T):
        a, b = 4 * int(offsets[t]), 4 * int(offsets[t + 1])
        if a == b:
            continue
        if b - a < MASK_WORDS:
            raise FormatError(f"tile {t}: shorter than its masks")
        bm, bk = divmod(t, KT)
        masks = words[a:a + MASK_WORDS].view(np.uint64)
        vals = words[a + MASK_WORDS:b].view(np.uint16)
        v = 0
        for g in range(8):
            for lane in range(64):
                m = int(masks[lane])
                for bit in range(8 * g, 8 * g + 8):
                    if not (m >> bit) & 1:
                        continue
                    r, c = position(lane, bit)
                    i, j = bm * TILE + r, bk * TILE + c
                    if i >= M or j >= K:
                        raise FormatError(f"tile {t}: bit outside the matrix")
                    if v >= vals.size:
                        raise FormatError(f"tile {t}: more mask bits than values")
                    A[i, j] = vals[v]
                    v += 1
        if v == 0 or (v + 7) // 8 * 8 != vals.size:
            raise FormatError(f"tile {t}: value count does not match its masks")
    return A


def format_bytes(mask: np.ndarray) -> int:
    """Blob bytes plus the offset array, from the per-tile kept counts (B3)."""
    M, K = mask.shape
    MB, KT, T = grid(M, K, TILE, TILE)
    total = 0
    for bm in range(MB):
        for bk in range(KT):
            total += tile_bytes(int((mask[bm * TILE:(bm + 1) * TILE, bk * TILE:(bk + 1) * TILE] != 0).sum()))
    return total + 4 * (T + 1)
