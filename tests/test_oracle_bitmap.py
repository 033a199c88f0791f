"""Pins for the oracle's bitmap-tile format (CPU only).

Tied to things other than itself: a hand-worked encoding (tests/golden/tiny_bitmap.json),
exhaustive round trips over every mask of a 3 x 3 matrix, agreement with the independent
Tiled-CSL decoder on the same inputs, the closed-form byte count, and rejection of
malformed blobs.
"""
import itertools
import json
import os

import numpy as np
import pytest

import lscd_synth as syn
from oracle import bitmap as ob
from oracle import tiled_csl as tc


def _bits(vals):
    return np.asarray(vals, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_golden_tiny_bitmap(golden_dir):
    with open(os.path.join(golden_dir, "tiny_bitmap.json")) as f:
        g = json.load(f)
    M, K = g["M"], g["K"]
    A16 = np.zeros((M, K), dtype=np.uint16)
    mask = np.zeros((M, K), dtype=np.uint8)
    for r, c, v in g["entries"]:
        A16[r, c] = _bits([v])[0]
        mask[r, c] = 1
    words, offs = ob.encode(A16, mask)
    assert [f"{w:08X}" for w in words] == g["words_hex"]
    assert offs.tolist() == g["offsets_16B"]
    assert ob.format_bytes(mask) == g["format_bytes"]
    assert np.array_equal(ob.decode(words, offs, M, K), tc.masked(A16, mask))


def test_positions_are_the_mfma_operand_layout():
    """Every (lane, bit) names a distinct tile position, and lane l's chunk g (8 bits) is the
    8 consecutive columns the 16x16x32 MFMA takes from lane l for row block g // 2 and k step
    g % 2: row 16 * (g // 2) + l % 16, columns 32 * (g % 2) + 8 * (l // 16) .. + 7."""
    seen = set()
    for lane in range(64):
        for bit in range(64):
            r, c = ob.position(lane, bit)
            assert 0 <= r < 64 and 0 <= c < 64 and (r, c) not in seen
            seen.add((r, c))
            assert ob.lane_bit(r, c) == (lane, bit)
            g = bit // 8
            assert r == 16 * (g // 2) + lane % 16
            assert c - bit % 8 == 32 * (g % 2) + 8 * (lane // 16)
    assert len(seen) == 4096


def test_every_mask_of_3x3_round_trips():
    vals = _bits(np.arange(1, 10).reshape(3, 3) * (-1.0) ** np.arange(9).reshape(3, 3))
    for bits in range(1 << 9):
        mask = np.array([(bits >> i) & 1 for i in range(9)], dtype=np.uint8).reshape(3, 3)
        words, offs = ob.encode(vals, mask)
        assert np.array_equal(ob.decode(words, offs, 3, 3), tc.masked(vals, mask)), bits
        assert words.size * 4 + 8 == ob.format_bytes(mask)


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.2), (130, 200, 0.5), (65, 129, 0.9), (100, 70, 0.05),
                                      (50, 90, 0.3), (7, 9, 1.0)])
def test_agrees_with_tiled_csl_decoder(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M * K)
    words, offs = ob.encode(case.A16, case.mask)
    tw, to = tc.encode_canonical(case.A16, case.mask, 64, 64)
    assert np.array_equal(ob.decode(words, offs, M, K), tc.decode(tw, to, M, K, 64, 64))


def test_byte_count_closed_forms():
    full = np.ones((64, 64), dtype=np.uint8)
    assert ob.format_bytes(full) == 512 + 2 * 4096 + 8          # masks + all values + 2 offsets
    assert ob.format_bytes(np.zeros((128, 64), dtype=np.uint8)) == 4 * 3
    one = np.zeros((64, 64), dtype=np.uint8)
    one[5, 7] = 1
    assert ob.format_bytes(one) == 512 + 16 + 8                 # one value padded to a 16-byte vector
    # at 50% density the blob is ~(2 * 0.5 + 1/8) bytes per element, against 4 * 0.5 for Tiled-CSL
    rng = np.random.default_rng(0)
    half = (rng.random((640, 640)) < 0.5).astype(np.uint8)
    assert abs(ob.format_bytes(half) / half.size - 1.125) < 0.01


def test_signed_zero_survives():
    A = np.array([[0x8000, 0x0000, 0x3C00]], dtype=np.uint16)
    mask = np.array([[1, 1, 0]], dtype=np.uint8)
    words, offs = ob.encode(A, mask)
    out = ob.decode(words, offs, 1, 3)
    assert out[0, 0] == 0x8000 and out[0, 1] == 0 and out[0, 2] == 0


def test_decoder_rejects_malformed():
    case = syn.random_case(70, 70, 1, 0.3, seed=3)
    words, offs = ob.encode(case.A16, case.mask)
    bad_last = offs.copy()
    bad_last[-1] += 1
    with pytest.raises(tc.FormatError):
        ob.decode(words, bad_last, 70, 70)
    # a mask bit outside the matrix: tile 1 covers columns 64..69 only; lane 16, bit 0 is
    # tile row 0, column 8 -> matrix column 72 >= K
    t1 = 4 * int(offs[1])
    bad2 = words.copy()
    bad2[t1 + 2 * 16] |= np.uint32(1)
    with pytest.raises(tc.FormatError):
        ob.decode(bad2, offs, 70, 70)
    # one more mask bit than stored values in a tile whose values fill their padding exactly
    with pytest.raises(tc.FormatError):
        full = np.ones((8, 8), dtype=np.uint8)
        w, o = ob.encode(case.A16[:8, :8], full)
        w[1] |= np.uint32(1 << 31)        # lane 0, bit 63: row 48, column 39 (outside the 8 x 8 matrix too)
        ob.decode(w, o, 8, 8)
    offs_bad = offs.copy()
    offs_bad[1], offs_bad[2] = offs[2], offs[1]
    with pytest.raises(tc.FormatError):
        ob.decode(words, offs_bad, 70, 70)
