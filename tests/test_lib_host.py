"""Host-side checks of liblscd.so (no GPU needed).

* the library loads and exports every entry point include/lscd.h declares;
* the host encoder (lscd_pack) agrees with the oracle's canonical encoding on what is
  unique -- the tile offsets and each tile's set of words -- and the rest is valid
  (padding words are copies, the oracle decodes it back to the masked matrix);
* lscd_import rejects invalid encodings before touching a device;
* argument errors are reported as statuses, not crashes.
"""
import os
import re

import numpy as np
import pytest

import lscd_synth as syn
import unstructured_sparse_skinny_amd as L
from oracle import tiled_csl as tc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "lscd.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(lscd_[a-z_]+)\s*\(", text))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(L._lib, name), name
    assert L.lscd_status_string(L.LSCD_ERROR_INVALID_FORMAT) == "invalid format"
    assert L.lscd_status_string(99) == "unknown status"


def _check_pack_against_oracle(A16, mask, tm=64, tk=64):
    words, offs = L.lscd_pack(A16, mask, tm, tk)
    m = mask if mask is not None else ((A16 & 0x7FFF) != 0).astype(np.uint8)
    ow, oo = tc.encode_canonical(A16, m, tm, tk)
    assert np.array_equal(offs, oo)                       # unique: per-tile padded counts
    assert words.size == ow.size
    for t, (a, b) in enumerate(zip(tc.tile_sets(words, offs), tc.tile_sets(ow, oo))):
        assert np.array_equal(a, b), t                    # unique: the set of entries per tile
    dec = tc.decode(words, offs, A16.shape[0], A16.shape[1], tm, tk)   # validity (duplicates agree)
    assert np.array_equal(dec, tc.masked(A16, m))
    return words, offs


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.2), (200, 333, 0.3), (1, 1, 1.0), (65, 129, 0.5),
                                      (130, 70, 0.0), (64, 200, 1.0), (300, 64 * 5 + 3, 0.1)])
def test_pack_matches_oracle(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M + K)
    _check_pack_against_oracle(case.A16, case.mask)


def test_pack_config1_and_null_mask():
    c = syn.make_config(1)
    _check_pack_against_oracle(c.A16, c.mask)
    # NULL mask keeps every entry whose value is not +-0
    A = c.A16.copy()
    A[c.mask == 0] = 0
    A[0, 0], A[0, 1] = 0x8000, 0x0000                    # -0 and +0 are dropped without a mask
    w, o = L.lscd_pack(A, None)
    m = ((A & 0x7FFF) != 0).astype(np.uint8)
    assert np.array_equal(o, tc.encode_canonical(A, m, 64, 64)[1])


def test_pack_other_tile_shapes():
    case = syn.random_case(100, 90, 1, 0.4, seed=3)
    for tm, tk in [(16, 16), (1, 256), (256, 256), (7, 13)]:
        _check_pack_against_oracle(case.A16, case.mask, tm, tk)


def test_pack_signed_zero_kept_by_mask():
    A = np.array([[0x8000, 0x0000, 0x3C00]], dtype=np.uint16)
    mask = np.array([[1, 1, 0]], dtype=np.uint8)
    words, offs = _check_pack_against_oracle(A, mask)
    assert sorted(words.tolist()) == sorted([0x00008000, 0x00010000, 0x00010000, 0x00010000]) or \
        set(words.tolist()) == {0x00008000, 0x00010000}


def test_reorder_spreads_banks():
    """The bank-aware order gives store instructions more distinct LDS banks than index order."""
    case = syn.random_case(64, 64, 1, 0.3, seed=1)

    def mean_distinct(words):
        nvec = words.size // 4
        vals = []
        for j in range((nvec + 63) // 64):
            L_ = min(64, nvec - 64 * j)
            for e in range(4):
                idx = words[4 * (64 * j + np.arange(L_)) + e] >> 16
                b = (idx * 2) ^ (((idx * 2) >> 3) & 0x70)
                vals.append(len(set(((b >> 2) & 31).tolist())) / min(L_, 32))
        return np.mean(vals)

    w_re, _ = L.lscd_pack(case.A16, case.mask)
    os.environ["LSCD_NO_REORDER"] = "1"
    try:
        w_plain, _ = L.lscd_pack(case.A16, case.mask)
    finally:
        del os.environ["LSCD_NO_REORDER"]
    assert mean_distinct(w_re) > mean_distinct(w_plain)


def test_import_rejects_invalid_formats():
    case = syn.random_case(100, 130, 1, 0.3, seed=8)
    words, offs = L.lscd_pack(case.A16, case.mask)
    M, K = case.M, case.K

    def expect_format_error(w, o, m=M, k=K):
        with pytest.raises(L.LSCDError) as ei:
            L.lscd_import(w, o, m, k)
        assert ei.value.status == L.LSCD_ERROR_INVALID_FORMAT

    o2 = offs.copy(); o2[-1] += 4
    expect_format_error(words, o2)                         # last offset != word count
    o3 = offs.copy(); o3[0] = 4
    expect_format_error(words, o3)                         # does not start at 0
    o4 = offs.copy(); o4[1] = o4[1] + 2
    expect_format_error(words, o4)                         # tile not a multiple of 4
    o5 = offs.copy(); o5[1], o5[2] = o5[2], o5[1]
    if o5[1] != o5[2]:
        expect_format_error(words, o5)                     # decreasing
    w = words.copy(); w[0] = (4096 << 16) | (w[0] & 0xFFFF)
    expect_format_error(w, offs)                           # index beyond the 64x64 tile
    # index inside the tile but outside the matrix: tile (0, 2) covers columns 128..129 only
    a, b = int(offs[2]), int(offs[3])
    assert b > a
    w = words.copy(); w[a] = (5 << 16) | 0x3C00            # row 0, in-tile column 5 -> column 133 >= K
    expect_format_error(w, offs)
    # conflicting duplicate inside one tile
    a, b = int(offs[0]), int(offs[1])
    if b - a >= 2:
        w = words.copy()
        w[a + 1] = (w[a] & 0xFFFF0000) | ((w[a] + 1) & 0xFFFF)
        expect_format_error(w, offs)


def test_argument_errors_are_statuses():
    A = np.zeros((4, 4), np.uint16)
    with pytest.raises(L.LSCDError) as ei:
        L.lscd_pack(A, None, 512, 256)                     # tile area > 65536
    assert ei.value.status == L.LSCD_ERROR_INVALID_VALUE
    with pytest.raises(L.LSCDError):
        L.lscd_pack(A, None, 0, 64)
    # too-short output arrays are refused by the C entry point
    st = L._lib.lscd_pack(A.ctypes.data, None, 4, 4, 2, 2, None, 0, None, 0)
    assert st == L.LSCD_ERROR_INVALID_VALUE
    # M or K above 2^30 is refused before A is read (the kernels index in 32 bits)
    nw, nt = L.ctypes.c_int64(), L.ctypes.c_int64()
    for M, K in ((2**30 + 1, 1), (1, 2**30 + 1), (2**31, 4)):
        st = L._lib.lscd_pack_size(A.ctypes.data, None, M, K, 64, 64, L.ctypes.byref(nw), L.ctypes.byref(nt))
        assert st == L.LSCD_ERROR_INVALID_VALUE, (M, K)
    h = L.ctypes.c_void_p()
    st = L._lib.lscd_import(None, 0, np.zeros(2, np.uint32).ctypes.data, 2**30 + 64, 64, 64, 64, L.ctypes.byref(h))
    assert st == L.LSCD_ERROR_INVALID_VALUE and not h.value
    assert L._lib.lscd_spmm(None, None, None, 16, None) == L.LSCD_ERROR_INVALID_VALUE
    assert L._lib.lscd_destroy(None) == L.LSCD_SUCCESS
    assert L._lib.lscd_get_info(None, None) == L.LSCD_ERROR_INVALID_VALUE


def test_linear_cost_model():
    """The selection model: sparse for skinny N at high sparsity, dense once N is large or the
    matrix is nearly dense; both estimates grow with N within each kernel regime, the sparse
    one with the stored words."""
    M, K = 12288, 12288
    T = (M // 64) * (K // 64)
    for keep, small_n_sparse in ((0.2, True), (0.5, None), (1.0, False)):
        nw = int(keep * M * K)
        ts, td = L.lscd_linear_model(M, K, nw, T, 8)
        if small_n_sparse is not None:
            assert (ts < td) == small_n_sparse, (keep, ts, td)
        ts_big, td_big = L.lscd_linear_model(M, K, nw, T, 4096)
        assert td_big < ts_big, keep                       # compute-bound: dense wins
        for regime in ((1, 8, 16, 32, 64), (65, 128, 256, 257, 1024)):   # skinny kernels / wide kernel
            prev = (0.0, 0.0)
            for N in regime:
                cur = L.lscd_linear_model(M, K, nw, T, N)
                assert cur[0] >= prev[0] and cur[1] >= prev[1], (keep, N)
                prev = cur
    a = L.lscd_linear_model(M, K, 10_000_000, T, 16)[0]
    b = L.lscd_linear_model(M, K, 20_000_000, T, 16)[0]
    assert b > a
    for bad in ((0, K, 0, T, 8), (M, K, -1, T, 8), (M, K, 0, T, 0)):
        with pytest.raises(L.LSCDError):
            L.lscd_linear_model(*bad)


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.2), (130, 200, 0.5), (1, 1, 1.0), (65, 129, 0.9), (100, 300, 0.0),
                                      (257, 700, 0.3)])
def test_pack_bitmap_matches_oracle(M, K, keep):
    """The bitmap layout is fully determined (no free order), so the host encoder must equal
    the oracle's encoding word for word."""
    from oracle import bitmap as ob
    case = syn.random_case(M, K, 1, keep, seed=M + 2 * K)
    words, offs = L.lscd_pack_bitmap(case.A16, case.mask)
    ow, oo = ob.encode(case.A16, case.mask)
    assert np.array_equal(offs, oo)
    assert np.array_equal(words, ow)
    A = case.A16.copy()
    A[case.mask == 0] = 0
    A[0, 0] = 0x8000                                         # -0 is dropped without a mask
    w2, o2 = L.lscd_pack_bitmap(A, None)
    m2 = ((A & 0x7FFF) != 0).astype(np.uint8)
    ow2, oo2 = ob.encode(A, m2)
    assert np.array_equal(w2, ow2) and np.array_equal(o2, oo2)


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.5), (130, 200, 0.5), (1, 1, 1.0), (65, 129, 0.9), (100, 300, 0.0),
                                      (257, 700, 0.45), (200, 130, 0.05), (128, 64, 1.0)])
def test_pack_three_level_matches_oracle(M, K, keep):
    """The three-level layout is fully determined (slot order, codes, residual order), so the
    host encoder must equal the oracle's encoding word for word."""
    from oracle import three_level as otl
    case = syn.random_case(M, K, 1, keep, seed=M + 5 * K)
    words, offs = L.lscd_pack_three_level(case.A16, case.mask)
    ow, oo = otl.encode(case.A16, case.mask)
    assert np.array_equal(offs, oo)
    assert np.array_equal(words, ow)
    A = case.A16.copy()
    A[case.mask == 0] = 0
    A[0, 0] = 0x8000                                         # -0 is dropped without a mask
    w2, o2 = L.lscd_pack_three_level(A, None)
    m2 = ((A & 0x7FFF) != 0).astype(np.uint8)
    ow2, oo2 = otl.encode(A, m2)
    assert np.array_equal(w2, ow2) and np.array_equal(o2, oo2)


def test_pack_three_level_size_and_errors():
    case = syn.random_case(100, 100, 1, 0.5, seed=1)
    words, offs = L.lscd_pack_three_level(case.A16, case.mask)
    assert offs.size == 5 and words.size == 4 * int(offs[-1]) and words.size >= 4 * 1280
    with pytest.raises(L.LSCDError):
        L.lscd_pack_three_level(np.zeros((0, 5), dtype=np.uint16), None)


@pytest.mark.parametrize("tm", [80, 96, 112, 128])
@pytest.mark.parametrize("M,K,keep", [(300, 200, 0.3), (129, 64 * 3 + 5, 1.0), (1, 1, 1.0), (500, 130, 0.05)])
def test_pack_tall_tiles_matches_oracle(tm, M, K, keep):
    """Taller tiles (the heights the product kernels run): same unique parts as the oracle's
    canonical encoding, valid padding, bank-aware order inside each tile."""
    case = syn.random_case(M, K, 1, keep, seed=M + K + tm)
    _check_pack_against_oracle(case.A16, case.mask, tm, 64)
