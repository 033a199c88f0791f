"""Oracle three-level format: 4:2 layer, slot-filling layer, residual layer.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the follow-up summary of the pages (gist.science, section "Metodologia", part 1
"Formato di Archiviazione a Tre Livelli").  The sparse matrix is split into three layers:

* a 4:2 layer ("Sparse-TC"): of every four consecutive weights of a row, two kept entries
  with 2-bit positions, the form the structured-sparse matrix instructions consume;
* a slot-filling layer: the kept entries a group of four cannot hold (its third and fourth)
  are moved into the slots the 4:2 layer leaves unused, and their positions are stored as
  4-bit distances to the previous moved entry ("Parallel Differential Distance"), with
  dummy points inserted where a distance would not fit;
* a residual layer for what is left, in a plain sparse list.

The summary gives no layout, no slot order and no sizes.  Readings taken here (T1..T7); the
layout follows the operand registers of the 16x16x64 structured-sparse MFMA, whose lane
mapping was measured on the hardware (see T2):

T1  Tiles of 64 x 64 in row-block-major order (t = bm * ceil(K/64) + bk), as in the
    Tiled-CSL format.  A tile with no kept entry stores nothing.
T2  Lane regions.  Within a tile, "operand" i (0..3) and lane l (0..63) own row
    16*i + (l % 16) and the 16 columns 16*(l // 16) .. +15, i.e. four groups of four
    columns.  Lane l's region is its four rows x 16 columns; region position
    p = 16*i + c, c = column - 16*(l // 16).
T3  4:2 layer.  Slot s (0..7) of operand i, lane l belongs to group s // 2.  The first two
    kept entries of a group (ascending column) take slots 2g and 2g+1 with their in-group
    positions (2 bits each).  A slot the group does not use holds +0 and the lowest
    in-group position that has no kept entry (different for the two slots of an empty group).
T4  Excess entries are the third and fourth kept entries of a group.  Within a lane region
    they are taken in ascending region position and placed, in slot order j = 8*i + s, into
    the region's unused slots.  Each placed entry costs one 4-bit code d - 1, where d is its
    distance to the previously placed entry (the first counts from position -1).  When the
    next entry is more than 16 positions away, a dummy point (value +0) is placed 16 positions
    on, taking a slot and a code.  A region has at most 8 codes.  Placement stops at the first
    entry (or dummy) that finds no free slot or code; that entry and all later excess entries
    of the region go to the residual layer.
T5  Residual layer: per tile, 32-bit words (fp16 bits | (r*64 + c) << 16) in ascending
    position, padded to a multiple of four words with copies of the last word (the
    Tiled-CSL reading R4).  The summary calls this layer CSR; with 64-row tiles and the row
    inside the word, a row-pointer array would repeat what the words hold.
T6  Tile blob (32-bit little-endian words): 1024 words of values (operand i, lane l: words
    4*(64*i + l) .. +3 hold slots 0..7, slot s in the low (even s) or high half of word s//2);
    then 256 words of per-lane metadata (lane l: words 1024 + 4*l .. +3 = positions of
    operands 0|1 (low|high 16 bits, 2 bits per slot), positions of operands 2|3, fill mask
    (bit j set <=> slot j holds a slot-filling entry or a dummy), codes (code k in bits
    4k..4k+3)); then the residual words.  Offsets: T+1 entries in 16-byte units.
T7  Entries at positions outside the matrix (edge tiles) can only be dummies or unused
    slots, always +0; a decoder drops them and rejects any other value there.
"""
from __future__ import annotations

import numpy as np

from .tiled_csl import FormatError, grid

TILE = 64
VALUE_WORDS = 1024                     # 4 operands x 64 lanes x 4 words
META_WORDS = 256                       # 64 lanes x 4 words
FIXED_WORDS = VALUE_WORDS + META_WORDS
MAX_CODES = 8


def lane_cell(l: int, i: int, g: int):
    """(row, first column) inside the tile of operand i, lane l, group g (T2)."""
    return 16 * i + (l % 16), 16 * (l // 16) + 4 * g


def _tile_lanes(sub_m: np.ndarray, sub_a: np.ndarray):
    """Per-lane layer contents of one tile (arrays padded to 64 x 64 with no kept entry)."""
    vals = np.zeros((4, 64, 8), dtype=np.uint16)
    pos = np.zeros((4, 64, 8), dtype=np.uint32)
    fill = np.zeros(64, dtype=np.uint32)
    codes = np.zeros(64, dtype=np.uint32)
    residual = []                     # (r*64 + c, value)
    stats = {"layer1": 0, "placed": 0, "dummies": 0, "residual": 0}
    for l in range(64):
        excess = []                   # (region position, row, col, value)
        unused = []                   # slot index j = 8*i + s
        for i in range(4):
            for g in range(4):
                r, c0 = lane_cell(l, i, g)
                kept = [c for c in range(4) if sub_m[r, c0 + c]]
                free = [c for c in range(4) if not sub_m[r, c0 + c]]
                for s in range(2):
                    if s < len(kept):
                        c = kept[s]
                        vals[i, l, 2 * g + s] = sub_a[r, c0 + c]
                        pos[i, l, 2 * g + s] = c
                        stats["layer1"] += 1
                    else:
                        # lowest free in-group position, distinct for the two slots of an empty group
                        pos[i, l, 2 * g + s] = free[s - len(kept)]
                        unused.append(8 * i + 2 * g + s)
                for c in kept[2:]:
                    excess.append((16 * i + 4 * g + c, r, c0 + c, int(sub_a[r, c0 + c])))
        excess.sort()
        prev, k, u = -1, 0, 0
        stopped = False
        for p, r, c, v in excess:
            if not stopped:
                while p - prev > 16:
                    if u >= len(unused) or k >= MAX_CODES:
                        stopped = True
                        break
                    j = unused[u]
                    u += 1
                    fill[l] |= np.uint32(1 << j)
                    codes[l] |= np.uint32(15 << (4 * k))
                    k += 1
                    prev += 16
                    stats["dummies"] += 1        # slot value stays +0
                if not stopped and (u >= len(unused) or k >= MAX_CODES):
                    stopped = True
            if stopped:
                residual.append((r * 64 + c, v))
                stats["residual"] += 1
                continue
            j = unused[u]
            u += 1
            fill[l] |= np.uint32(1 << j)
            codes[l] |= np.uint32((p - prev - 1) << (4 * k))
            k += 1
            prev = p
            vals[j // 8, l, j % 8] = v
            stats["placed"] += 1
    return vals, pos, fill, codes, sorted(residual), stats


def _tile_blob(vals, pos, fill, codes, residual) -> np.ndarray:
    words = np.zeros(FIXED_WORDS, dtype=np.uint32)
    words[:VALUE_WORDS] = vals.reshape(-1).view(np.uint32)
    idx16 = np.zeros((4, 64), dtype=np.uint32)
    for s in range(8):
        idx16 |= pos[:, :, s] << (2 * s)
    meta = words[VALUE_WORDS:].reshape(64, 4)
    meta[:, 0] = idx16[0] | (idx16[1] << 16)
    meta[:, 1] = idx16[2] | (idx16[3] << 16)
    meta[:, 2] = fill
    meta[:, 3] = codes
    if residual:
        rw = [np.uint32(v) | (np.uint32(p) << 16) for p, v in residual]
        while len(rw) % 4:
            rw.append(rw[-1])
        words = np.concatenate([words, np.asarray(rw, dtype=np.uint32)])
    return words


def encode(A16: np.ndarray, mask: np.ndarray, with_stats: bool = False):
    """Three-level encoding of (A16, mask): (words uint32[total], offsets uint32[T+1]) per T1-T7."""
    M, K = A16.shape
    MB, KT, _ = grid(M, K, TILE, TILE)
    chunks, offs = [], [0]
    total = {"layer1": 0, "placed": 0, "dummies": 0, "residual": 0}
    for bm in range(MB):
        for bk in range(KT):
            r0, c0 = bm * TILE, bk * TILE
            sm = np.zeros((TILE, TILE), dtype=bool)
            sa = np.zeros((TILE, TILE), dtype=np.uint16)
            blk = mask[r0:r0 + TILE, c0:c0 + TILE] != 0
            sm[:blk.shape[0], :blk.shape[1]] = blk
            sa[:blk.shape[0], :blk.shape[1]] = A16[r0:r0 + TILE, c0:c0 + TILE]
            if not sm.any():
                offs.append(offs[-1])
                continue
            vals, pos, fill, codes, residual, st = _tile_lanes(sm, sa)
            for key in total:
                total[key] += st[key]
            blob = _tile_blob(vals, pos, fill, codes, residual)
            chunks.append(blob)
            offs.append(offs[-1] + blob.size // 4)
    words = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.uint32)
    out = (words.astype(np.uint32), np.asarray(offs, dtype=np.uint32))
    return out + (total,) if with_stats else out


def decode(words: np.ndarray, offsets: np.ndarray, M: int, K: int) -> np.ndarray:
    """Dense fp16 bit patterns of a three-level encoding; raises FormatError when it is not valid.

    Layers are applied as slot filling, residual, then the 4:2 layer: the +0 of a dummy point
    may sit where the 4:2 layer holds an entry, and the 4:2 layer writes last.
    """
    words = np.asarray(words, dtype=np.uint32)
    offsets = np.asarray(offsets, dtype=np.int64)
    MB, KT, T = grid(M, K, TILE, TILE)
    if offsets.shape != (T + 1,) or offsets[0] != 0 or np.any(np.diff(offsets) < 0):
        raise FormatError("offsets must be non-decreasing from 0 with T+1 entries")
    if 4 * offsets[-1] != words.size:
        raise FormatError("last offset must match the blob size")
    A = np.zeros((M, K), dtype=np.uint16)

    def put(t_r0, t_c0, r, c, v, what):
        i, j = t_r0 + r, t_c0 + c
        if i >= M or j >= K:
            if v != 0:
                raise FormatError(f"{what}: value outside the matrix")
            return
        A[i, j] = v

    for t in range(T):
        a, b = 4 * int(offsets[t]), 4 * int(offsets[t + 1])
        if a == b:
            continue
        if b - a < FIXED_WORDS:
            raise FormatError(f"tile {t}: shorter than its fixed part")
        bm, bk = divmod(t, KT)
        r0, c0 = bm * TILE, bk * TILE
        tw = words[a:b]
        vals = tw[:VALUE_WORDS].view(np.uint16).reshape(4, 64, 8)
        meta = tw[VALUE_WORDS:FIXED_WORDS].reshape(64, 4)
        res = tw[FIXED_WORDS:]
        pos = np.zeros((4, 64, 8), dtype=np.uint32)
        for i in range(4):
            half = (meta[:, i // 2] >> (16 * (i % 2))) & 0xFFFF
            for s in range(8):
                pos[i, :, s] = (half >> (2 * s)) & 3
        # slot filling
        for l in range(64):
            fill, codes = int(meta[l, 2]), int(meta[l, 3])
            n = bin(fill).count("1")
            if n > MAX_CODES:
                raise FormatError(f"tile {t} lane {l}: more filled slots than codes")
            prev = -1
            for k, j in enumerate(jj for jj in range(32) if (fill >> jj) & 1):
                p = prev + ((codes >> (4 * k)) & 15) + 1
                if p >= 64:
                    raise FormatError(f"tile {t} lane {l}: slot-filling position past the region")
                prev = p
                r, c = 16 * (p // 16) + l % 16, 16 * (l // 16) + p % 16
                put(r0, c0, r, c, int(vals[j // 8, l, j % 8]), f"tile {t} lane {l} code {k}")
        # residual
        for w in res:
            pp = int(w) >> 16
            if pp >= TILE * TILE:
                raise FormatError(f"tile {t}: residual position out of the tile")
            put(r0, c0, pp // TILE, pp % TILE, int(w) & 0xFFFF, f"tile {t} residual")
        # 4:2 layer (slots not filled)
        for l in range(64):
            fill = int(meta[l, 2])
            for i in range(4):
                for s in range(8):
                    if (fill >> (8 * i + s)) & 1:
                        continue
                    r, c = lane_cell(l, i, s // 2)
                    put(r0, c0, r, c + int(pos[i, l, s]), int(vals[i, l, s]), f"tile {t} lane {l} slot {s}")
    return A


def format_bytes(A16: np.ndarray, mask: np.ndarray) -> int:
    """Blob bytes plus the offset array."""
    words, offs = encode(A16, mask)
    return 4 * words.size + 4 * offs.size
