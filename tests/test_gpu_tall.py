"""GPU parity for tiles taller than 64 rows (80, 96, 112, 128 x 64).

lscd_encode picks the tile height per matrix (lscd_default_tile_m); these tests force
every height on small and ragged shapes so that each kernel family runs with it:
  * the decoded matrix is bit-exact;
  * integer-valued products are bit-exact for N across the kernel boundaries (8-wavefront
    independent variant up to 32 columns, shared B tile up to 64, wide kernel above) with
    forced K splits;
  * Gaussian products pass the tolerance gates;
  * the device encoder builds the same words as the host encoder for the chosen height;
  * the height choice itself: 112 rows for the OPT-30B MLP1 and OPT-66B QKV shapes on a
    256-CU device, 64 where 64-row blocks do not fill the GPU.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from oracle import tiled_csl as tc
from tests._util import assert_gates, env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L

HEIGHTS = [80, 96, 112, 128]


def encode(A16, mask, tm):
    w, o = L.lscd_pack(A16, mask, tm, 64)
    return L.lscd_import(w, o, A16.shape[0], A16.shape[1], tm, 64)


def run(h, B16, M):
    B = torch.from_numpy(np.ascontiguousarray(B16).view(np.float16)).to("cuda")
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    L.lscd_spmm(h, B, C)
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("tm", HEIGHTS)
@pytest.mark.parametrize("M,K,keep", [(300, 520, 0.3), (1, 1, 1.0), (129, 200, 1.0), (700, 1111, 0.2)])
def test_tall_decode_bit_exact(tm, M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M + K + tm)
    h = encode(case.A16, case.mask, tm)
    say(f"tall decode tm={tm} M={M} K={K} R={h.info['reg_vectors']}")
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    L.lscd_debug_decode(h, A)
    torch.cuda.synchronize()
    assert np.array_equal(A.cpu().numpy().view(np.uint16), tc.masked(case.A16, case.mask))


@pytest.mark.parametrize("tm", HEIGHTS)
@pytest.mark.parametrize("N", [1, 16, 32, 33, 64, 65, 200])
@pytest.mark.parametrize("splits", [None, "3"])
def test_tall_integer_bit_exact(tm, N, splits):
    case = syn.random_case(333, 1000 + 8 * N, N, 0.35, seed=N + tm, values="int3")
    with env(LSCD_SPLITK=splits):
        h = encode(case.A16, case.mask, tm)
    say(f"tall int tm={tm} N={N} S={h.info['splits']} Sw={h.info['splits_wide']} variant={h.info['variant']}")
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.abs(C64).max() < 2048
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(C64))


@pytest.mark.parametrize("tm", HEIGHTS)
@pytest.mark.parametrize("N", [8, 32, 64, 128])
def test_tall_gaussian_within_tolerance(tm, N):
    case = syn.random_case(1000, 1111, N, 0.25, seed=tm * N)
    h = encode(case.A16, case.mask, tm)
    say(f"tall gauss tm={tm} N={N}")
    assert_gates(run(h, case.B16, case.M), osp.spmm_f64(case.A16, case.mask, case.B16), f"tm={tm} N={N}")


def test_tall_dense_tile_past_the_stage():
    """Full 128 x 64 tiles (8192 words) exceed the largest staging stage: the rest path."""
    case = syn.random_case(256, 200, 16, 1.0, seed=3, values="int3")
    h = encode(case.A16, case.mask, 128)
    assert h.info["max_tile_words"] == 128 * 64 and h.info["reg_vectors"] == 12
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16)))


def test_default_tile_height_choice():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"cus={cus}")
    if cus == 256:
        assert L.lscd_default_tile_m(28672, 7168) == 112
        assert L.lscd_default_tile_m(27648, 9216) == 112
        assert L.lscd_default_tile_m(49152, 12288) == 64   # 768 blocks of 64: already 3 per CU
    assert L.lscd_default_tile_m(12288, 49152) == 64       # 192 blocks: K splits balance
    assert L.lscd_default_tile_m(1, 1) == 64
    with env(LSCD_TILE_M="96"):
        assert L.lscd_default_tile_m(1000, 1000) == 96


def test_tall_device_encoder_matches_host():
    case = syn.random_case(700, 1111, 1, 0.3, seed=8)
    Ad = torch.from_numpy(case.A16.view(np.float16)).to("cuda")
    md = torch.from_numpy(case.mask.astype(np.uint8)).to("cuda")
    for tm in HEIGHTS:
        with env(LSCD_TILE_M=str(tm)):
            assert L.lscd_default_tile_m(case.M, case.K) == tm
            h = L.lscd_encode_device(Ad, md)
        assert h.info["tile_m"] == tm
        words, offs = L.lscd_export(h)
        pw, po = L.lscd_pack(case.A16, case.mask, tm, 64)
        assert np.array_equal(offs, po) and np.array_equal(words, pw), tm


@pytest.mark.parametrize("tm,keep", [(112, 0.6), (80, 1.0)])
@pytest.mark.parametrize("splits", [None, "3"])
def test_tall_overflow_n64_runs_wide_kernel(tm, keep, splits):
    """Tall tiles denser than the shared-B register stage: N = 33..64 runs the N > 64 kernel
    (variant 3, N padded to 128, splits of its first launch width); N <= 32 keeps the
    8-wavefront kernel.  Integer products bit-exact for N on both sides of the boundaries."""
    case = syn.random_case(300, 700, 64, keep, seed=tm, values="int3")
    with env(LSCD_SPLITK=splits):
        h = encode(case.A16, case.mask, tm)
    info = h.info
    say(f"overflow tm={tm} keep={keep} maxw={info['max_tile_words']} R={info['reg_vectors']} "
        f"variant={info['variant']} S={info['splits']} Sw={info['splits_wide']}")
    assert info["max_tile_words"] > info["reg_vectors"] * 64 * 4
    assert info["variant"][:2] == [2, 2] and info["variant"][2] == 3
    assert info["splits"][2] == info["splits_wide"][0]
    for N in (16, 32, 33, 48, 64):
        B16 = case.B16[:N]
        C64 = osp.spmm_f64(case.A16, case.mask, B16)
        assert np.abs(C64).max() < 2048
        assert np.array_equal(run(h, B16, case.M), osp.fp16_rne(C64)), f"N={N}"


def test_tall_fitting_tiles_keep_shared_b():
    """Tall tiles that fit the register stage keep the shared-B kernel at N = 64."""
    case = syn.random_case(300, 700, 64, 0.35, seed=5, values="int3")
    h = encode(case.A16, case.mask, 112)
    assert h.info["max_tile_words"] <= h.info["reg_vectors"] * 64 * 4
    assert h.info["variant"][2] in (0, 6)   # shared B, four or three row blocks per workgroup
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16)))
