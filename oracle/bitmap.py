"""Oracle bitmap-tile format: encoder, validating decoder and byte count.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the follow-up summary of the pages (gist.science, section "Problematica",
third point): CSR-like position metadata costs as much as the values at about 50%
sparsity, and a bitmap (one bit per position) cuts that metadata at the price of
more decoding work on chip.  The pages give no layout; the readings taken here:

B1  tiles and tile order as in the Tiled-CSL format (row-block-major,
    t = bm * ceil(K/tile_k) + bk), tile_k <= 64 so one row of a tile fits a 64-bit
    mask.
B2  a tile with at least one kept entry stores tile_m 64-bit row masks (bit c of
    mask r set <=> entry (r, c) of the tile is kept; positions outside the matrix are
    0), little-endian, followed by the kept fp16 bit patterns in row-major order,
    padded with 0x0000 to a multiple of 8 values (whole 16-byte vectors).  A tile
    with no kept entry stores nothing.
B3  the offset array has T+1 entries counted in 16-byte units, offsets[0] = 0.
    The blob is handled as 32-bit little-endian words: the mask of row r is words
    2r (low half) and 2r + 1 (high half); value v of the tile is the low (v even) or
    high (v odd) 16 bits of word 2*tile_m + v // 2.
B4  the mask decides what is stored, as in the Tiled-CSL reading R5 (a kept +0 or
    -0 is stored, and -0 survives the round trip).
"""
from __future__ import annotations

import numpy as np

from .tiled_csl import FormatError, grid


def tile_bytes(n_kept: int, tm: int = 64) -> int:
    """Bytes of one tile: masks + values rounded up to 8 (B2); 0 for an empty tile."""
    if n_kept == 0:
        return 0
    return 8 * tm + 16 * ((n_kept + 7) // 8)


def encode(A16: np.ndarray, mask: np.ndarray, tm: int = 64, tk: int = 64):
    """Bitmap encoding of (A16, mask): (words uint32[total], offsets uint32[T+1]) per B1-B4."""
    if tk > 64:
        raise ValueError("tile_k must be <= 64 (one 64-bit mask per tile row)")
    M, K = A16.shape
    MB, KT, _ = grid(M, K, tm, tk)
    chunks, offs = [], [0]
    for bm in range(MB):
        for bk in range(KT):
            r0, c0 = bm * tm, bk * tk
            sub_m = mask[r0:r0 + tm, c0:c0 + tk] != 0
            sub_a = A16[r0:r0 + tm, c0:c0 + tk]
            n = int(sub_m.sum())
            if n == 0:
                offs.append(offs[-1])
                continue
            masks = np.zeros(tm, dtype=np.uint64)
            for r in range(sub_m.shape[0]):
                bits = 0
                for c in range(sub_m.shape[1]):
                    if sub_m[r, c]:
                        bits |= 1 << c
                masks[r] = bits
            vals = sub_a[sub_m]                       # boolean indexing is row-major
            nv = (n + 7) // 8 * 8
            padded = np.zeros(nv, dtype=np.uint16)
            padded[:n] = vals
            blob = np.concatenate([masks.view(np.uint32), padded.view(np.uint32)])
            chunks.append(blob)
            offs.append(offs[-1] + blob.size // 4)
    words = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.uint32)
    return words.astype(np.uint32), np.asarray(offs, dtype=np.uint32)


def decode(words: np.ndarray, offsets: np.ndarray, M: int, K: int, tm: int = 64, tk: int = 64) -> np.ndarray:
    """Dense fp16 bit patterns of a bitmap encoding; raises FormatError when it is not valid."""
    words = np.asarray(words, dtype=np.uint32)
    offsets = np.asarray(offsets, dtype=np.int64)
    MB, KT, T = grid(M, K, tm, tk)
    if offsets.shape != (T + 1,) or offsets[0] != 0 or np.any(np.diff(offsets) < 0):
        raise FormatError("offsets must be non-decreasing from 0 with T+1 entries")
    if 4 * offsets[-1] != words.size:
        raise FormatError("last offset must match the blob size")
    A = np.zeros((M, K), dtype=np.uint16)
    for t in range(T):
        a, b = 4 * int(offsets[t]), 4 * int(offsets[t + 1])
        if a == b:
            continue
        bm, bk = divmod(t, KT)
        rows = min(tm, M - bm * tm)
        cols = min(tk, K - bk * tk)
        if b - a < 2 * tm:
            raise FormatError(f"tile {t}: shorter than its masks")
        masks = words[a:a + 2 * tm].view(np.uint64)
        vals = words[a + 2 * tm:b].view(np.uint16)
        n = 0
        for r in range(tm):
            m = int(masks[r])
            for c in range(64):
                if (m >> c) & 1:
                    if r >= rows or c >= cols:
                        raise FormatError(f"tile {t}: bit outside the matrix")
                    if n >= vals.size:
                        raise FormatError(f"tile {t}: more mask bits than values")
                    A[bm * tm + r, bk * tk + c] = vals[n]
                    n += 1
        if n == 0 or (n + 7) // 8 * 8 != vals.size:
            raise FormatError(f"tile {t}: value count does not match its masks")
    return A


def format_bytes(mask: np.ndarray, tm: int = 64, tk: int = 64) -> int:
    """Blob bytes plus the offset array, from the per-tile kept counts (B2, B3)."""
    M, K = mask.shape
    MB, KT, T = grid(M, K, tm, tk)
    total = 0
    for bm in range(MB):
        for bk in range(KT):
            total += tile_bytes(int((mask[bm * tm:(bm + 1) * tm, bk * tk:(bk + 1) * tk] != 0).sum()), tm)
    return total + 4 * (T + 1)
