"""Pins for the plain C oracle (oracle/spmm_loop.c: Tiled-CSL decode and the fp64 triple loop).

CPU only.  It is pinned to things outside itself:
  * the hand-worked golden example (words, offsets, dense A and C);
  * every one of the 65536 fp16 bit patterns, converted against the hardware conversion of
    numpy (exact in fp64), through a 1 x 1 product with B = 1;
  * the closed form of integer inputs (int64 matrix product) -- bit-identical;
  * the Python oracle's decode (encodings shuffled and padded) and its invalid-format rules;
  * exact rational sums on tiny inputs, and the fp64 product of a library routine on Gaussian
    inputs within the rounding of fp64 sums.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import lscd_synth as syn
from oracle import loop
from oracle import spmm as osp
from oracle import tiled_csl as tc


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "tiny_tiled_csl.json")) as f:
        return json.load(f)


def test_golden_decode_and_product(golden_dir):
    g = _golden(golden_dir)
    words = np.array([int(x, 16) for x in g["canonical_words_hex"]], dtype=np.uint32)
    offs = np.array(g["offsets"], dtype=np.uint32)
    A16 = np.asarray(g["A"], np.float64).astype(np.float16).view(np.uint16)
    mask = np.asarray(g["mask"], np.uint8)
    dense = loop.decode(words, offs, g["M"], g["K"], g["tile_m"], g["tile_k"])
    assert np.array_equal(dense, tc.masked(A16, mask))
    B16 = np.asarray(g["B"], np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(loop.spmm(dense, B16), np.asarray(g["C"], np.float64))


def test_every_fp16_pattern_converts_exactly():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(-1, 1)
    one = np.array([[0x3C00]], dtype=np.uint16)
    got = loop.spmm(bits, one)[0]
    want = bits[:, 0].view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # (a sum starts at +0, so -0 * 1 comes out as +0: the sign of a zero is not observable here)


@pytest.mark.parametrize("seed", range(4))
def test_integer_closed_form_bit_identical(seed):
    case = syn.random_case(150 + 37 * seed, 700 + 91 * seed, 1 + 7 * seed, keep=0.35, seed=seed, values="int3")
    A = tc.masked(case.A16, case.mask)
    a = np.asarray(A).view(np.float16).astype(np.int64)
    b = case.B16.view(np.float16).astype(np.int64)
    exact = (b @ a.T).astype(np.float64)
    got = loop.spmm(A, case.B16)
    assert np.array_equal(got, exact)
    assert np.array_equal(got, osp.spmm_f64(case.A16, case.mask, case.B16))


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, N = (int(x) for x in rng.integers(1, 6, size=3))
    case = syn.random_case(M, K, N, keep=0.6, seed=seed, values="unit")
    A = tc.masked(case.A16, case.mask)
    got = loop.spmm(A, case.B16)
    exact = osp.spmm_exact_small(case.A16, case.mask, case.B16)
    a = osp.fp16_to_f64(A)
    b = osp.fp16_to_f64(case.B16)
    for n in range(N):
        for i in range(M):
            bound = float(np.abs(a[i]) @ np.abs(b[n])) * 2.0 ** -50
            assert abs(Fraction(float(got[n, i])) - exact[n][i]) <= Fraction(bound)


def test_gaussian_matches_library_product_within_fp64_rounding():
    case = syn.random_case(300, 2000, 16, keep=0.3, seed=9)
    got = loop.spmm(tc.masked(case.A16, case.mask), case.B16, rows=np.arange(0, 300, 7))
    want = osp.spmm_f64(case.A16, case.mask, case.B16, rows=np.arange(0, 300, 7))
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


@pytest.mark.parametrize("M,K,tm,tk", [(3, 5, 2, 4), (130, 200, 64, 64), (257, 70, 112, 64), (50, 50, 7, 9)])
def test_decode_matches_python_oracle_on_shuffled_padded_encodings(M, K, tm, tk):
    case = syn.random_case(M, K, 1, keep=0.4, seed=M + K)
    words, offs = tc.encode_canonical(case.A16, case.mask, tm, tk)
    rng = np.random.default_rng(1)
    w2 = words.copy()
    for t in range(offs.size - 1):
        seg = w2[offs[t]:offs[t + 1]]
        rng.shuffle(seg)
    dense = loop.decode(w2, offs, M, K, tm, tk)
    assert np.array_equal(dense, tc.decode(w2, offs, M, K, tm, tk))
    assert np.array_equal(dense, tc.masked(case.A16, case.mask))


def test_decode_rejects_what_the_python_oracle_rejects():
    case = syn.random_case(20, 20, 1, keep=0.5, seed=3)
    words, offs = tc.encode_canonical(case.A16, case.mask, 8, 8)
    bad = []
    o = offs.copy(); o[0] = 4; bad.append((words, o))                       # does not start at 0
    o = offs.copy(); o[2], o[3] = o[3], o[2]; bad.append((words, o))       # decreasing
    o = offs.copy(); o[1] += 1; bad.append((words, o))                      # not a multiple of 4
    bad.append((words[:-4], offs))                                          # total != word count
    w = words.copy(); w[0] = (w[0] & 0xFFFF) | (64 << 16); bad.append((w, offs))   # outside the tile
    w = words.copy(); t_last = offs.size - 2
    w[offs[t_last]] = (w[offs[t_last]] & 0xFFFF) | ((7 * 8 + 7) << 16)              # outside A (edge tile)
    bad.append((w, offs))
    w = words.copy(); w[1] = (w[0] & 0xFFFF0000) | ((w[0] + 1) & 0xFFFF); bad.append((w, offs))  # conflict
    for w_, o_ in bad:
        with pytest.raises(ValueError):
            loop.decode(w_, o_, 20, 20, 8, 8)
        with pytest.raises(tc.FormatError):
            tc.decode(w_, o_, 20, 20, 8, 8)


def test_rows_subset_and_threads():
    case = syn.random_case(97, 300, 5, keep=0.3, seed=11, values="int3")
    A = tc.masked(case.A16, case.mask)
    full = loop.spmm(A, case.B16, threads=1)
    rows = np.array([96, 0, 50, 50, 3])
    assert np.array_equal(loop.spmm(A, case.B16, rows=rows, threads=3), full[:, rows])
    assert loop.max_threads() >= 1
