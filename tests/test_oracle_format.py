"""Pins for the oracle's Tiled-CSL encoder/decoder (CPU only).

Each pin ties the oracle to something other than itself: hand-worked
encodings of the format definition (tests/golden), exhaustive brute force over
every mask of tiny matrices, and the format's own invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import tiled_csl as tc


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _bits(vals):
    return np.asarray(vals, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_golden_tiny_encode_decode(golden_dir):
    g = _load(golden_dir, "tiny_tiled_csl.json")
    A16 = _bits(g["A"])
    mask = np.asarray(g["mask"], dtype=np.uint8)
    words, offs = tc.encode_canonical(A16, mask, g["tile_m"], g["tile_k"])
    assert [f"{w:08X}" for w in words] == g["canonical_words_hex"]
    assert offs.tolist() == g["offsets"]
    dec = tc.decode(words, offs, g["M"], g["K"], g["tile_m"], g["tile_k"])
    assert np.array_equal(dec, tc.masked(A16, mask))


def test_golden_signed_zero_and_edge_tile(golden_dir):
    g = _load(golden_dir, "signed_zero_tiled_csl.json")
    A16 = np.array([[int(h, 16) for h in row] for row in g["A_bits_hex"]], dtype=np.uint16)
    mask = np.asarray(g["mask"], dtype=np.uint8)
    words, offs = tc.encode_canonical(A16, mask, g["tile_m"], g["tile_k"])
    assert [f"{w:08X}" for w in words] == g["canonical_words_hex"]
    assert offs.tolist() == g["offsets"]
    dec = tc.decode(words, offs, g["M"], g["K"], g["tile_m"], g["tile_k"])
    want = np.array([[int(h, 16) for h in row] for row in g["decoded_bits_hex"]], dtype=np.uint16)
    assert np.array_equal(dec, want)


@pytest.mark.parametrize("shape,tile", [((3, 3), (2, 2)), ((4, 4), (3, 3)), ((4, 4), (1, 4))])
def test_brute_force_every_mask_round_trips(shape, tile):
    """Every mask of a tiny matrix (full and ragged edge tiles) round-trips bit-exactly."""
    M, K = shape
    tm, tk = tile
    rng = np.random.default_rng(3)
    # distinct nonzero values (and one explicit -0) so a misplaced word always shows
    A16 = (np.arange(1, M * K + 1, dtype=np.float64).reshape(M, K) * 0.25).astype(np.float16).view(np.uint16)
    A16[0, 0] = 0x8000
    MB, KT, T = tc.grid(M, K, tm, tk)
    for bits in range(1 << (M * K)):
        mask = ((bits >> np.arange(M * K)) & 1).astype(np.uint8).reshape(M, K)
        words, offs = tc.encode_canonical(A16, mask, tm, tk)
        # tile word counts are the padded popcounts of the mask inside each tile
        for t in range(T):
            bm, bk = divmod(t, KT)
            n = int(mask[bm * tm:(bm + 1) * tm, bk * tk:(bk + 1) * tk].sum())
            assert offs[t + 1] - offs[t] == (n + 3) // 4 * 4
        dec = tc.decode(words, offs, M, K, tm, tk)
        assert np.array_equal(dec, tc.masked(A16, mask)), bits
        if bits % 4093 == 0:       # a shuffled tile order inside tiles decodes the same
            w2 = words.copy()
            for t in range(T):
                seg = w2[offs[t]:offs[t + 1]]
                rng.shuffle(seg)
            assert np.array_equal(tc.decode(w2, offs, M, K, tm, tk), dec)


def test_random_matrix_round_trip_and_shuffle():
    rng = np.random.default_rng(11)
    M, K, tm, tk = 203, 517, 64, 64
    A16 = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    mask = (rng.random((M, K)) < 0.23).astype(np.uint8)
    words, offs = tc.encode_canonical(A16, mask, tm, tk)
    assert np.array_equal(tc.decode(words, offs, M, K, tm, tk), tc.masked(A16, mask))
    w2 = words.copy()
    for t in range(offs.size - 1):
        rng.shuffle(w2[offs[t]:offs[t + 1]])
    assert np.array_equal(tc.decode(w2, offs, M, K, tm, tk), tc.masked(A16, mask))
    # nnz accounting: distinct words per tile = kept positions in the tile
    assert sum(s.size for s in tc.tile_sets(words, offs)) == int(mask.sum())


def test_empty_and_full():
    M, K = 70, 130
    A16 = np.full((M, K), 0x3C00, dtype=np.uint16)
    words, offs = tc.encode_canonical(A16, np.zeros((M, K), np.uint8), 32, 64)
    assert words.size == 0 and not offs.any()
    assert not tc.decode(words, offs, M, K, 32, 64).any()
    words, offs = tc.encode_canonical(A16, np.ones((M, K), np.uint8), 32, 64)
    assert np.array_equal(tc.decode(words, offs, M, K, 32, 64), A16)


def _small():
    A16 = _bits([[1.0, 2.0, 0.0, 3.0], [0.0, 5.0, 6.0, 0.0]])
    mask = (A16 != 0).astype(np.uint8)
    return A16, mask, tc.encode_canonical(A16, mask, 2, 2)


def test_decode_rejects_invalid_formats():
    A16, mask, (words, offs) = _small()
    M, K = A16.shape
    assert np.array_equal(tc.decode(words, offs, M, K, 2, 2), A16)
    # conflicting duplicate: a padding word that changes the value
    w = words.copy()
    w[3] = (w[3] & 0xFFFF0000) | 0x4400
    if (words[3] & 0xFFFF) != 0x4400:
        with pytest.raises(tc.FormatError):
            tc.decode(w, offs, M, K, 2, 2)
    # index outside the tile
    w = words.copy()
    w[0] = (4 << 16) | (w[0] & 0xFFFF)
    with pytest.raises(tc.FormatError):
        tc.decode(w, offs, M, K, 2, 2)
    # non-decreasing offsets / multiples of 4 / end marker
    with pytest.raises(tc.FormatError):
        tc.decode(words, np.array([0, 8, 4, 8], dtype=np.uint32)[:offs.size], M, K, 2, 2)
    o = offs.copy()
    o[1] += 1
    with pytest.raises(tc.FormatError):
        tc.decode(words, o, M, K, 2, 2)
    with pytest.raises(tc.FormatError):
        tc.decode(words[:-4], offs, M, K, 2, 2)


def test_decode_rejects_position_outside_matrix():
    # 3x3 matrix, 2x2 tiles: the edge tile (1,1) covers only (2,2); index 1 -> (2,3) is outside
    A16 = np.zeros((3, 3), np.uint16)
    mask = np.zeros((3, 3), np.uint8)
    words, offs = tc.encode_canonical(A16, mask, 2, 2)
    offs = np.array([0, 0, 0, 0, 4], dtype=np.uint32)
    bad = np.full(4, (1 << 16) | 0x3C00, dtype=np.uint32)
    with pytest.raises(tc.FormatError):
        tc.decode(bad, offs, 3, 3, 2, 2)
    good = np.full(4, (0 << 16) | 0x3C00, dtype=np.uint32)
    dec = tc.decode(good, offs, 3, 3, 2, 2)
    assert dec[2, 2] == 0x3C00 and dec.sum() == 0x3C00


def test_plausible_encoder_mistakes_fail_the_golden(golden_dir):
    """A transposed in-tile index or swapped word halves would not reproduce the golden words."""
    g = _load(golden_dir, "tiny_tiled_csl.json")
    words = np.array([int(h, 16) for h in g["canonical_words_hex"]], dtype=np.uint32)
    swapped = ((words & 0xFFFF) << 16) | (words >> 16)
    with pytest.raises(tc.FormatError):
        tc.decode(swapped, np.array(g["offsets"]), g["M"], g["K"], g["tile_m"], g["tile_k"])
    # column-major in-tile index would place (1,1) [idx 5 row-major] at idx 3: different word
    A16 = _bits(g["A"])
    mask = np.asarray(g["mask"], dtype=np.uint8)
    w, _ = tc.encode_canonical(A16.T.copy(), mask.T.copy(), g["tile_k"], g["tile_m"])
    assert [f"{x:08X}" for x in w] != g["canonical_words_hex"]


def test_tile_limit():
    with pytest.raises(ValueError):
        tc.encode_canonical(np.zeros((2, 2), np.uint16), np.zeros((2, 2), np.uint8), 512, 256)
