"""lscd_spmm_noalloc: the product with its split-K partial sums in the library's static per-GPU
array instead of the handle's workspace (for callers that cannot allocate).

Called through the C ABI and checked against the oracle's gates and against lscd_spmm on the same
handle: the same kernels and plan, so the results are bit-identical.  The first call on each
handle is lscd_spmm_noalloc, before anything has written the handle's own workspace, and a last
call follows an lscd_spmm of another product: neither that workspace's contents nor its absence
may show in the result.  Two problems in a row, the second smaller, show that the array's
left-over contents do not matter; a plan whose partials exceed the array is refused with
NOT_SUPPORTED.
"""
import ctypes

import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from tests._util import assert_gates, env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L


def _call(fn, h, B16, M):
    B = torch.from_numpy(np.ascontiguousarray(B16).view(np.float16)).to("cuda")
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    st = fn(ctypes.c_void_p(h.ptr), ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(C.data_ptr()), B16.shape[0],
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, C.cpu().numpy().view(np.uint16)


def _both(h, case):
    # first on a fresh handle, whose own workspace no call has written yet
    st1, got = _call(L._lib.lscd_spmm_noalloc, h, case.B16, case.M)
    assert st1 == L.LSCD_SUCCESS, st1
    assert_gates(got, osp.spmm_f64(case.A16, case.mask, case.B16), case.name)
    st0, ref = _call(L._lib.lscd_spmm, h, case.B16, case.M)
    assert st0 == L.LSCD_SUCCESS, st0
    assert np.array_equal(got, ref)
    # the handle's workspace now holds the partial sums of another product (B with its signs
    # flipped); lscd_spmm_noalloc must neither read them nor be disturbed by them
    st2, neg = _call(L._lib.lscd_spmm, h, case.B16 ^ np.uint16(0x8000), case.M)
    assert st2 == L.LSCD_SUCCESS and not np.array_equal(neg, ref)
    st3, again = _call(L._lib.lscd_spmm_noalloc, h, case.B16, case.M)
    assert st3 == L.LSCD_SUCCESS and np.array_equal(again, ref)


@pytest.mark.parametrize("fmt", ["tiled-csl", "bitmap", "three-level"])
def test_noalloc_matches_lscd_spmm_twice_second_smaller(fmt):
    enc = {"tiled-csl": L.lscd_encode, "bitmap": L.lscd_encode_bitmap, "three-level": L.lscd_encode_three_level}[fmt]
    big = syn.random_case(1100, 4096, 64, 0.35, seed=21, name="big")
    small = syn.random_case(300, 1000, 8, 0.3, seed=22, name="small")
    with env(LSCD_SPLITK="4"):
        hb = enc(big.A16, big.mask)
    with env(LSCD_SPLITK="2"):
        hs = enc(small.A16, small.mask)
    say(f"noalloc {fmt}: big splits={hb.info['splits']} small splits={hs.info['splits']}")
    assert max(hb.info["splits"]) > 1 and max(hs.info["splits"]) > 1
    _both(hb, big)
    _both(hs, small)


def test_noalloc_wide_and_unsplit():
    case = syn.random_case(700, 3000, 200, 0.3, seed=23, name="wide")
    with env(LSCD_SPLITK="3"):
        h = L.lscd_encode(case.A16, case.mask)
    say(f"noalloc wide: splits_wide={h.info['splits_wide']}")
    _both(h, case)
    one = syn.random_case(130, 300, 16, 0.3, seed=24, name="one")
    with env(LSCD_SPLITK="1"):
        h1 = L.lscd_encode(one.A16, one.mask)
    _both(h1, one)


def test_noalloc_refuses_partials_beyond_the_array():
    case = syn.random_case(49152, 512, 64, 0.05, seed=25, name="tall")
    with env(LSCD_SPLITK="8"):
        h = L.lscd_encode(case.A16, case.mask)
    S = h.info["splits"][2]
    say(f"noalloc refuse: splits={h.info['splits']}")
    assert S * 64 * case.M * 4 > 64 << 20
    st, _ = _call(L._lib.lscd_spmm_noalloc, h, case.B16, case.M)
    assert st == L.LSCD_ERROR_NOT_SUPPORTED
    st, C = _call(L._lib.lscd_spmm, h, case.B16, case.M)
    assert st == L.LSCD_SUCCESS
    rows = np.arange(0, case.M, 97)
    assert_gates(C[:, rows], osp.spmm_f64(case.A16, case.mask, case.B16, rows=rows), "lscd_spmm")
