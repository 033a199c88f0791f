"""Pins of the three-level oracle (oracle/three_level.py) to facts outside its own code.

* Hand-worked tiles: one lane region with two excess entries in one group and a far one
  (dummy points bridge the gap), one that runs out of codes (the ninth point goes to the
  residual words); the expected words are derived by hand from readings T2-T6.
* Counting: the 4:2 layer holds min(count, 2) entries of every group of four and the excess
  is max(count - 2, 0), computed here by array reshaping, not by the oracle's loops; placed +
  residual = excess.
* Closed form: for an i.i.d. Bernoulli(1/2) mask the expected excess per group is
  P(3) + 2 P(4) = 6/16 of 2 expected kept entries, so 18.75% of the kept entries (the
  summary quotes about 17.7% for real weights).
* Dense tiles: every group has 4 entries, so no slot is free and every excess entry is a
  residual word: 1280 + 2048 words per tile.
* Round trip bit-exact (signed zeros included) on ragged shapes and densities 0..1, and the
  decoder's rejections.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import three_level as tl
from oracle.tiled_csl import FormatError


def masked(A16, mask):
    return np.where(mask != 0, A16, 0).astype(np.uint16)


def one_tile(entries):
    """64 x 64 A and mask with the given {(r, c): value_bits}."""
    A = np.zeros((64, 64), dtype=np.uint16)
    m = np.zeros((64, 64), dtype=np.uint8)
    for (r, c), v in entries.items():
        A[r, c] = v
        m[r, c] = 1
    return A, m


def lane_meta(words, lane):
    return words[tl.VALUE_WORDS + 4 * lane: tl.VALUE_WORDS + 4 * lane + 4]


def slot_value(words, lane, j):
    i, s = divmod(j, 8)
    w = int(words[4 * (64 * i + lane) + s // 2])
    return (w >> (16 * (s % 2))) & 0xFFFF


def test_hand_worked_dummy_points():
    # lane 0 owns rows 0, 16, 32, 48 and columns 0..15 (region position p = 16*i + c)
    ent = {(0, 0): 0x3C00, (0, 1): 0x4000, (0, 2): 0x4200, (0, 3): 0x4400,   # group 0 full: excess p = 2, 3
           (32, 5): 0x4500,                                                 # one entry in group 1 of row 32
           (48, 12): 0x4600, (48, 13): 0x4700, (48, 14): 0x4800}            # excess p = 48 + 14 = 62
    A, m = one_tile(ent)
    words, offs, st = tl.encode(A, m, with_stats=True)
    assert list(offs) == [0, 320] and words.size == 1280
    assert st == {"layer1": 5, "placed": 3, "dummies": 3, "residual": 0}
    idx01, idx23, fill, codes = (int(x) for x in lane_meta(words, 0))
    # unused slots in order: row 0 groups 1-3 -> j = 2..7 (the first six points take them)
    assert fill == 0xFC
    # points: p=2 (code 2), p=3 (code 0), dummies at 19, 35, 51 (code 15 each), p=62 (code 10)
    assert codes == 2 | (0 << 4) | (15 << 8) | (15 << 12) | (15 << 16) | (10 << 20)
    assert [slot_value(words, 0, j) for j in range(2, 8)] == [0x4200, 0x4400, 0, 0, 0, 0x4800]
    assert [slot_value(words, 0, j) for j in (0, 1)] == [0x3C00, 0x4000]
    # positions: row 0 group 0 uses (0, 1); unused groups take their lowest free positions (0, 1)
    assert idx01 & 0xFFFF == 0x4444
    # row 32 (operand 2): group 1 holds column 5 -> slot 2 position 1, slot 3 the lowest free (0)
    assert (idx23 >> (2 * 2)) & 3 == 1 and (idx23 >> (2 * 3)) & 3 == 0
    # row 48 (operand 3): group 3 holds columns 12, 13 in the 4:2 layer
    assert (idx23 >> 16 >> 12) & 0xF == 0b0100
    assert slot_value(words, 0, 8 * 3 + 6) == 0x4600 and slot_value(words, 0, 8 * 3 + 7) == 0x4700
    for lane in range(1, 64):
        assert list(lane_meta(words, lane)[2:]) == [0, 0]
    assert np.array_equal(tl.decode(words, offs, 64, 64), masked(A, m))


def test_hand_worked_code_budget():
    ent = {}
    for i in (0, 1):                      # rows 0 and 16: three entries in each group -> 8 excess
        for g in range(4):
            for c in range(3):
                ent[(16 * i, 4 * g + c)] = 0x3C00 + 16 * i + 4 * g + c
    for c in range(3):                    # row 32 group 0: a ninth excess entry at p = 34
        ent[(32, c)] = 0x5000 + c
    A, m = one_tile(ent)
    words, offs, st = tl.encode(A, m, with_stats=True)
    assert st["placed"] == 8 and st["dummies"] == 0 and st["residual"] == 1
    _, _, fill, codes = (int(x) for x in lane_meta(words, 0))
    # unused slots: row 32 groups 1-3 (j = 18..23), then row 48 (j = 24..31); eight are used
    assert fill == sum(1 << j for j in range(18, 26))
    assert codes == 0x33333332            # p = 2, 6, 10, ..., 30: distances 3, 4, 4, ... minus one
    res = words[1280:]
    assert res.size == 4 and all(int(w) == 0x5002 | ((32 * 64 + 2) << 16) for w in res)
    assert np.array_equal(tl.decode(words, offs, 64, 64), masked(A, m))


@pytest.mark.parametrize("keep", [0.2, 0.5, 0.8])
def test_layer_counts_by_reshaping(keep):
    case = syn.random_case(128, 192, 1, keep, seed=int(keep * 10))
    words, offs, st = tl.encode(case.A16, case.mask, with_stats=True)
    cnt = (case.mask != 0).reshape(128, 48, 4).sum(axis=2)
    assert st["layer1"] == int(np.minimum(cnt, 2).sum())
    assert st["placed"] + st["residual"] == int(np.maximum(cnt - 2, 0).sum())
    assert st["layer1"] + st["placed"] + st["residual"] == int((case.mask != 0).sum())


def test_excess_fraction_closed_form():
    rng = np.random.default_rng(2024)
    M = K = 512
    mask = (rng.random((M, K)) < 0.5).astype(np.uint8)
    A16 = np.full((M, K), 0x3C00, dtype=np.uint16)
    _, _, st = tl.encode(A16, mask, with_stats=True)
    nnz = int(mask.sum())
    frac = (st["placed"] + st["residual"]) / nnz
    # per group: E[excess] = 6/16, sd of the excess count = sqrt(4*1/16 + 4*1/16 - (6/16)^2); 65536 groups
    sd = np.sqrt((4 / 16 + 4 / 16 - (6 / 16) ** 2) / 65536) / 2
    assert abs(frac - 0.1875) < 5 * sd + 1e-3


def test_dense_tiles_all_excess_residual():
    A16 = np.arange(128 * 64, dtype=np.uint32).astype(np.uint16).reshape(128, 64) | 0x0400
    mask = np.ones((128, 64), dtype=np.uint8)
    words, offs, st = tl.encode(A16, mask, with_stats=True)
    assert st == {"layer1": 4096, "placed": 0, "dummies": 0, "residual": 4096}
    assert list(offs) == [0, (1280 + 2048) // 4, 2 * (1280 + 2048) // 4]
    assert np.array_equal(tl.decode(words, offs, 128, 64), A16)


def test_no_excess_is_plain_four_two_compression():
    rng = np.random.default_rng(5)
    M, K = 64, 64
    mask = np.zeros((M, K), dtype=np.uint8)
    for r in range(M):
        for g in range(16):
            for c in rng.choice(4, rng.integers(0, 3), replace=False):
                mask[r, 4 * g + c] = 1
    A16 = (rng.integers(1, 0x7BFF, size=(M, K))).astype(np.uint16)
    words, offs = tl.encode(A16, mask)
    assert words.size == 1280
    meta = words[tl.VALUE_WORDS:].reshape(64, 4)
    assert not meta[:, 2].any() and not meta[:, 3].any()
    # slots: the kept values of each group in column order, zero padded to two
    vals = words[:tl.VALUE_WORDS].view(np.uint16).reshape(4, 64, 8)
    for l in range(64):
        for i in range(4):
            r, q = 16 * i + l % 16, l // 16
            for g in range(4):
                cols = [16 * q + 4 * g + c for c in range(4) if mask[r, 16 * q + 4 * g + c]]
                want = [A16[r, c] for c in cols] + [0] * (2 - len(cols))
                assert list(vals[i, l, 2 * g: 2 * g + 2]) == want


@pytest.mark.parametrize("M,K,keep", [(1, 1, 1.0), (63, 65, 0.5), (100, 130, 0.3), (130, 200, 0.6),
                                      (64, 64, 0.0), (70, 70, 0.95), (200, 100, 0.05)])
def test_round_trip_bit_exact(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M + 3 * K)
    A16 = case.A16.copy()
    A16[(np.arange(M)[:, None] + np.arange(K)[None, :]) % 7 == 0] = 0x8000   # kept -0 survives
    words, offs = tl.encode(A16, case.mask)
    assert np.array_equal(tl.decode(words, offs, M, K), masked(A16, case.mask))


def test_decoder_rejections():
    case = syn.random_case(100, 100, 1, 0.5, seed=4)
    words, offs = tl.encode(case.A16, case.mask)
    with pytest.raises(FormatError):
        tl.decode(words[:-4], offs, 100, 100)
    bad = offs.copy()
    bad[1] = 100                             # tile shorter than its fixed part
    bad[2:] = bad[2:] - (offs[1] - 100)
    with pytest.raises(FormatError):
        tl.decode(words[: 4 * int(bad[-1])], bad, 100, 100)
    w = words.copy()
    w[tl.VALUE_WORDS + 2] = 0xFFFFFFFF       # lane 0: 32 filled slots, more than the codes
    with pytest.raises(FormatError):
        tl.decode(w, offs, 100, 100)
    w = words.copy()
    w[tl.VALUE_WORDS + 2] = 0xFF             # eight points of distance 16 walk past the region
    w[tl.VALUE_WORDS + 3] = 0xFFFFFFFF
    with pytest.raises(FormatError):
        tl.decode(w, offs, 100, 100)
    # the last row block has rows 64..99; lane 36 of operand 3 is row 52 -> 116 >= 100: outside
    t = (1 * 2 + 1)
    a = 4 * int(offs[t])
    w = words.copy()
    lane = 36
    meta = w[a + tl.VALUE_WORDS + 4 * lane: a + tl.VALUE_WORDS + 4 * lane + 4]
    assert meta[2] == 0
    w[a + 4 * (64 * 3 + lane)] = 0x3C00       # a nonzero slot value outside the matrix
    with pytest.raises(FormatError):
        tl.decode(w, offs, 100, 100)
