"""Oracle Tiled-CSL format: canonical encoder and validating decoder.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: Flash-LLM paper review (xllm-io), section 3, "Tiled-CSL sparse encoding
format", and the component table of the same section.  The pages fix:

* the matrix A[M][K] is split into a grid of tiles and the format is laid out
  tile by tile;
* every nonzero is one 32-bit word made of a 16-bit value and a 16-bit index;
* the index is the nonzero's position within its tile;
* a per-tile offset array locates each tile's run of words;
* tiles are fetched with 128-bit (4-word) vector loads;
* inside a tile, the order of the nonzeros is a free choice (the pages reorder
  them ahead of time only to spread shared-memory bank accesses).

Readings taken where the pages are silent (all are also listed in the design
notes of the repository):

R1  word bits: value (fp16 bit pattern) in bits [15:0], index in bits [31:16].
R2  index: row-major position inside the tile, r * tile_k + c, so
    tile_m * tile_k <= 65536.
R3  tile order: row-block-major, t = bm * ceil(K/tile_k) + bk.  The offset array
    has T+1 entries, counted in 32-bit words, offsets[0] = 0, offsets[T] = total.
R4  padding for 4-word vector loads: a tile with n nonzeros holds
    round_up(n, 4) words; the extra words are exact copies of a real word of the
    same tile (rewriting a value is harmless, a fake (0, index 0) word would
    clobber a real entry at index 0).  An empty tile holds no words.
R5  the mask decides what is stored: a kept position is stored even if its
    value is +0 or -0; positions beyond M or K in edge tiles are never stored.
R6  the order of words inside a tile carries no meaning; the canonical encoder
    here uses ascending index and pads with copies of the last word.
"""
from __future__ import annotations

import numpy as np


class FormatError(ValueError):
    """The arrays do not form a valid Tiled-CSL encoding."""


def grid(M: int, K: int, tile_m: int, tile_k: int):
    """(row blocks, k blocks, tiles) of the tile grid."""
    MB = -(-M // tile_m)
    KT = -(-K // tile_k)
    return MB, KT, MB * KT


def masked(A16: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """A with every dropped position set to +0.0 (bits 0x0000); kept bits unchanged."""
    return np.where(mask.astype(bool), A16, np.uint16(0)).astype(np.uint16)


def _check_tile(tile_m: int, tile_k: int):
    if tile_m < 1 or tile_k < 1 or tile_m * tile_k > 65536:
        raise ValueError("tile must satisfy 1 <= tile_m * tile_k <= 65536 (16-bit in-tile index)")


def encode_canonical(A16: np.ndarray, mask: np.ndarray, tile_m: int, tile_k: int):
    """Encode (A, mask) into (words uint32[], offsets uint32[T+1]), canonical order.

    Steps in the order the format is described: walk the tiles in row-block-major
    order; within a tile gather each kept position's (in-tile index, value); append
    the tile's words; record where each tile starts.  Then pad each tile (R4).
    """
    _check_tile(tile_m, tile_k)
    M, K = A16.shape
    MB, KT, T = grid(M, K, tile_m, tile_k)
    ii, jj = np.nonzero(mask)                        # row-major order of kept positions
    ii = ii.astype(np.int64)
    jj = jj.astype(np.int64)
    tile = (ii // tile_m) * KT + (jj // tile_k)
    index = (ii % tile_m) * tile_k + (jj % tile_k)
    value = A16[ii, jj].astype(np.int64)
    order = np.lexsort((index, tile))                # by tile, then ascending in-tile index
    tile, index, value = tile[order], index[order], value[order]
    word = ((index << 16) | value).astype(np.uint32)

    count = np.bincount(tile, minlength=T).astype(np.int64)
    padded = (count + 3) // 4 * 4
    offsets = np.zeros(T + 1, dtype=np.int64)
    np.cumsum(padded, out=offsets[1:])
    if offsets[-1] >= 2 ** 32:
        raise ValueError("encoding exceeds 2^32 words")
    words = np.empty(int(offsets[-1]), dtype=np.uint32)
    real_start = np.zeros(T + 1, dtype=np.int64)
    np.cumsum(count, out=real_start[1:])
    # real words: position within tile = rank since the tile's first real word
    rank = np.arange(word.size, dtype=np.int64) - np.repeat(real_start[:-1], count)
    words[np.repeat(offsets[:-1], count) + rank] = word
    # padding words: copies of the tile's last real word
    npad = padded - count
    has_pad = np.nonzero(npad)[0]
    if has_pad.size:
        reps = npad[has_pad]
        dst = np.repeat(offsets[has_pad] + count[has_pad], reps) + (
            np.arange(int(reps.sum())) - np.repeat(np.cumsum(reps) - reps, reps))
        words[dst] = np.repeat(word[real_start[has_pad + 1] - 1], reps)
    return words, offsets.astype(np.uint32)


def decode(words: np.ndarray, offsets: np.ndarray, M: int, K: int, tile_m: int, tile_k: int,
           row_blocks=None) -> np.ndarray:
    """Turn an encoding back into dense A bits [M][K]; raise FormatError if invalid.

    Start from an all +0.0 matrix; for every tile, for every word of the tile,
    split the word into value and in-tile index, map the index to (row, column)
    of A, and write the value there.  Two words that land on the same position
    must carry the same bits (padding copies); otherwise the encoding is rejected.

    `row_blocks`, if given, is an iterable of row-block numbers: only those are
    decoded (the rest of the result stays +0.0), which bounds memory for large A.
    """
    _check_tile(tile_m, tile_k)
    words = np.asarray(words, dtype=np.uint32)
    offsets = np.asarray(offsets, dtype=np.int64)
    MB, KT, T = grid(M, K, tile_m, tile_k)
    if offsets.shape != (T + 1,):
        raise FormatError(f"offset array must have T+1 = {T + 1} entries")
    if offsets[0] != 0 or offsets[-1] != words.size:
        raise FormatError("offsets must start at 0 and end at the word count")
    count = np.diff(offsets)
    if np.any(count < 0):
        raise FormatError("offsets must be non-decreasing")
    if np.any(count % 4):
        raise FormatError("every tile must hold a multiple of 4 words")
    A = np.zeros((M, K), dtype=np.uint16)
    blocks = range(MB) if row_blocks is None else row_blocks
    for bm in blocks:
        lo, hi = int(offsets[bm * KT]), int(offsets[(bm + 1) * KT])
        w = words[lo:hi].astype(np.int64)
        bk = np.repeat(np.arange(KT, dtype=np.int64), count[bm * KT:(bm + 1) * KT])
        value = w & 0xFFFF
        index = w >> 16
        if np.any(index >= tile_m * tile_k):
            raise FormatError("in-tile index out of the tile")
        i = bm * tile_m + index // tile_k
        j = bk * tile_k + index % tile_k
        if np.any(i >= M) or np.any(j >= K):
            raise FormatError("word addresses a position outside A")
        flat = (i - bm * tile_m) * K + j
        order = np.argsort(flat, kind="stable")
        f_s, v_s = flat[order], value[order]
        same = f_s[1:] == f_s[:-1]
        if np.any(same & (v_s[1:] != v_s[:-1])):
            raise FormatError("two words write different values to one position")
        rows = A[bm * tile_m: min(M, (bm + 1) * tile_m)].reshape(-1)
        rows[f_s] = v_s.astype(np.uint16)
    return A


def tile_sets(words: np.ndarray, offsets: np.ndarray):
    """Per tile, the sorted array of distinct words (the order-free content of the tile)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    return [np.unique(words[offsets[t]:offsets[t + 1]]) for t in range(offsets.size - 1)]
