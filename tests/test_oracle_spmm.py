"""Pins for the oracle's fp64 product (CPU only).

The oracle's product is pinned against: a hand-worked example (tests/golden),
exact rational arithmetic by nested loops on tiny inputs, the closed form of
integer inputs (computed with integer arithmetic), column selection by an
identity-like B, and the all-zero result of a fully pruned matrix.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from oracle import tiled_csl as tc


def test_golden_tiny_product(golden_dir):
    with open(os.path.join(golden_dir, "tiny_tiled_csl.json")) as f:
        g = json.load(f)
    A16 = np.asarray(g["A"], np.float64).astype(np.float16).view(np.uint16)
    B16 = np.asarray(g["B"], np.float64).astype(np.float16).view(np.uint16)
    mask = np.asarray(g["mask"], np.uint8)
    C = osp.spmm_f64(A16, mask, B16)
    assert C.shape == (2, 3)
    assert np.array_equal(C, np.asarray(g["C"], np.float64))
    # the mask matters: dropping the mask (keeping nothing) gives zeros
    assert not osp.spmm_f64(A16, np.zeros_like(mask), B16).any()


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    M, K, N = rng.integers(1, 6, size=3)
    case = syn.random_case(int(M), int(K), int(N), keep=0.6, seed=seed, values="unit")
    C = osp.spmm_f64(case.A16, case.mask, case.B16)
    exact = osp.spmm_exact_small(case.A16, case.mask, case.B16)
    a = osp.fp16_to_f64(case.A16) * case.mask
    b = osp.fp16_to_f64(case.B16)
    for n in range(N):
        for i in range(M):
            bound = float(np.abs(a[i]) @ np.abs(b[n])) * 2.0 ** -50
            assert abs(Fraction(float(C[n, i])) - exact[n][i]) <= Fraction(bound)


def test_integer_closed_form_at_scale():
    """A, B integers in [-3,3]: every product and sum is an integer, exactly computed by int64 matmul."""
    case = syn.random_case(333, 2117, 19, keep=0.3, seed=5, values="int3")
    C = osp.spmm_f64(case.A16, case.mask, case.B16)
    a = osp.fp16_to_f64(case.A16).astype(np.int64) * case.mask.astype(np.int64)
    b = osp.fp16_to_f64(case.B16).astype(np.int64)
    exact = b @ a.T
    assert np.array_equal(C, exact.astype(np.float64))
    # rows subset = the same rows of the full result
    rows = np.array([0, 5, 332, 100])
    assert np.array_equal(osp.spmm_f64(case.A16, case.mask, case.B16, rows=rows), C[:, rows])
    # bit-exact rounding of integers to fp16 (|C| <= 2048 here is exact in fp16)
    assert np.abs(exact).max() < 2048
    assert np.array_equal(osp.fp16_rne(C).view(np.float16).astype(np.int64), exact)


def test_identity_b_selects_columns():
    case = syn.random_case(150, 97, 1, keep=0.4, seed=9)
    cols = [0, 96, 31, 50, 50, 7]
    B16 = syn.identity_B(case.K, cols)
    C = osp.spmm_f64(case.A16, case.mask, B16)
    Am = osp.fp16_to_f64(tc.masked(case.A16, case.mask))
    for n, c in enumerate(cols):
        assert np.array_equal(C[n], Am[:, c])


def test_fully_pruned_gives_exact_zero():
    case = syn.random_case(64, 200, 8, keep=0.0, seed=2)
    assert case.nnz == 0
    C = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.array_equal(osp.fp16_rne(C), np.zeros((8, 64), np.uint16))   # +0.0 bits


def test_dense_case_matches_rational_and_integer_paths():
    """At 0% sparsity the oracle is the plain dense product (checked by exact integer arithmetic)."""
    case = syn.random_case(40, 300, 7, keep=1.0, seed=4, values="int3")
    assert case.nnz == 40 * 300
    a = osp.fp16_to_f64(case.A16).astype(np.int64)
    b = osp.fp16_to_f64(case.B16).astype(np.int64)
    assert np.array_equal(osp.spmm_f64(case.A16, case.mask, case.B16), (b @ a.T).astype(np.float64))


def test_transposed_operand_would_fail():
    """Swapping the roles of M and N (a transposed operand) changes the hand-worked result."""
    A16 = np.asarray([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]).astype(np.float16).view(np.uint16)
    B16 = np.asarray([[1.0, -1.0]]).astype(np.float16).view(np.uint16)
    C = osp.spmm_f64(A16, np.ones((3, 2), np.uint8), B16)
    assert C.tolist() == [[-1.0, -1.0, -1.0]]
    B16 = np.asarray([[2.0, 1.0]]).astype(np.float16).view(np.uint16)
    assert osp.spmm_f64(A16, np.ones((3, 2), np.uint8), B16).tolist() == [[4.0, 10.0, 16.0]]


def test_fp16_rne_ties_and_overflow():
    # 1 + 2^-11 is halfway between 1 and 1+2^-10: ties to even -> 1.0
    assert osp.fp16_rne(np.array([1.0 + 2.0 ** -11]))[0] == 0x3C00
    # 1 + 3*2^-11 is halfway between 1+2^-10 and 1+2^-9: ties to even -> 1+2^-9
    assert osp.fp16_rne(np.array([1.0 + 3 * 2.0 ** -11]))[0] == 0x3C02
    assert osp.fp16_rne(np.array([70000.0]))[0] == 0x7C00
    assert osp.fp16_rne(np.array([-0.0]))[0] == 0x8000
