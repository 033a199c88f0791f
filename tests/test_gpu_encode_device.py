"""GPU parity of the device encoder (lscd_encode_device).

The format is integer work, so the bar is bit-exact: the device-built words and tile
offsets must equal the host encoder's (lscd_pack: same bank-aware order inside every
tile), the handle's counts must agree, and the oracle must decode the device words back
to the masked matrix.  Covered: ragged and single-entry matrices, empty and full tiles, no
mask (signed zeros dropped), the natural order (LSCD_NO_REORDER=1), and the full OPT-30B
MLP1 shape, whose products from the two handles must also be bit-identical.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import tiled_csl as tc
from tests._util import env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to("cuda")


def check_same(A16, mask):
    Ad = dev16(A16)
    md = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to("cuda")
    h = L.lscd_encode_device(Ad, md)
    tm = L.lscd_default_tile_m(*A16.shape)
    assert h.info["tile_m"] == tm
    words, offs = L.lscd_export(h)
    pw, po = L.lscd_pack(A16, mask, tm, 64)
    assert np.array_equal(offs, po)
    assert np.array_equal(words, pw)
    info, hh = h.info, L.lscd_encode(A16, mask).info
    for k in ("nnz", "nnz_padded", "max_tile_words", "num_tiles", "reg_vectors", "splits", "splits_wide"):
        assert info[k] == hh[k], k
    m = mask if mask is not None else ((A16 & 0x7FFF) != 0).astype(np.uint8)
    assert np.array_equal(tc.decode(words, offs, A16.shape[0], A16.shape[1], tm, 64), tc.masked(A16, m))
    return h


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.2), (130, 200, 0.5), (1, 1, 1.0), (65, 129, 0.9), (300, 70, 0.05),
                                      (200, 300, 1.0), (100, 300, 0.0), (257, 3000, 0.4), (1000, 1111, 0.25)])
def test_device_encoder_matches_host(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M * 3 + K)
    say(f"encode_device M={M} K={K} keep={keep}")
    check_same(case.A16, case.mask)


def test_device_encoder_null_mask_and_natural_order():
    case = syn.random_case(190, 260, 1, 0.4, seed=5)
    A = case.A16.copy()
    A[case.mask == 0] = 0
    A[0, 0], A[0, 1], A[5, 7] = 0x8000, 0x0000, 0x8000       # signed zeros are dropped without a mask
    check_same(A, None)
    with env(LSCD_NO_REORDER="1"):
        check_same(case.A16, case.mask)


def test_device_encoder_full_size_cfg2():
    case = syn.make_config(2)
    say(f"encode_device {case.name}")
    h = check_same(case.A16, case.mask)
    hh = L.lscd_encode(case.A16, case.mask)
    B = dev16(case.B16)
    C1 = torch.empty((case.N, case.M), dtype=torch.float16, device="cuda")
    C2 = torch.empty_like(C1)
    L.lscd_spmm(h, B, C1)
    L.lscd_spmm(hh, B, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def test_device_encoder_errors():
    A = torch.zeros(8, 9, dtype=torch.float16, device="cuda")
    h = L.ctypes.c_void_p()
    st = L._lib.lscd_encode_device(L.ctypes.c_void_p(A.data_ptr() + 1), None, 2, 2, None, L.ctypes.byref(h))
    assert st == L.LSCD_ERROR_INVALID_VALUE
    st = L._lib.lscd_encode_device(L.ctypes.c_void_p(A.data_ptr()), None, 0, 2, None, L.ctypes.byref(h))
    assert st == L.LSCD_ERROR_INVALID_VALUE
