"""GPU parity of the bitmap-tile path (lscd_encode_bitmap + lscd_spmm / lscd_debug_decode).

Bit-exact: the decoded matrix, the exported blob against the host encoder, fully dense tiles,
full chunks at odd starts, integer-valued products for N across the 16 / 32 / 64-column launch
boundaries with forced K splits.  Tolerance gates (tests/_util.py) for Gaussian inputs on
ragged shapes and, with sampled rows, at full OPT shapes.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import bitmap as ob
from oracle import spmm as osp
from oracle import tiled_csl as tc
from tests._util import assert_gates, env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to("cuda")


def run(h, B16, M):
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    L.lscd_spmm(h, dev(B16), C)
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint16)


SHAPES = [(64, 64, 0.3), (256, 256, 0.2), (300, 520, 0.3), (1000, 1111, 0.25), (1, 1, 1.0), (65, 70, 0.6),
          (512, 4096, 0.1), (257, 3000, 0.5), (200, 300, 1.0), (100, 300, 0.0)]


@pytest.mark.parametrize("M,K,keep", SHAPES)
def test_bitmap_decode_and_export_bit_exact(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M * 5 + K)
    say(f"bitmap decode M={M} K={K} keep={keep}")
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    assert h.info["format"] == 1 and h.info["nnz"] == int(case.mask.sum()) and h.info["reg_vectors"] == 0
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    L.lscd_debug_decode(h, A)
    torch.cuda.synchronize()
    assert np.array_equal(A.cpu().numpy().view(np.uint16), tc.masked(case.A16, case.mask))
    words, offs = L.lscd_export(h)
    ow, oo = ob.encode(case.A16, case.mask)
    assert np.array_equal(words, ow) and np.array_equal(offs, oo)


@pytest.mark.parametrize("N", [16, 32, 64])
def test_bitmap_full_tiles_bit_exact(N):
    # every position kept: all 16 groups of every lane hold 4 values
    case = syn.random_case(200, 300, N, 1.0, seed=2, values="int3")
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    say(f"bitmap dense N={N}")
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(C64))


@pytest.mark.parametrize("N", [1, 8, 16, 17, 32, 33, 64, 100])
@pytest.mark.parametrize("splits", [None, "1", "3"])
def test_bitmap_integer_bit_exact(N, splits):
    case = syn.random_case(333, 1000 + 8 * N, N, 0.35, seed=N + 77, values="int3")
    with env(LSCD_SPLITK=splits):
        h = L.lscd_encode_bitmap(case.A16, case.mask)
    say(f"bitmap int N={N} S={h.info['splits']}")
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.abs(C64).max() < 2048
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(C64))


@pytest.mark.parametrize("M,K,keep", SHAPES[:8])
@pytest.mark.parametrize("N", [8, 16, 32, 64])
def test_bitmap_gaussian_within_tolerance(M, K, keep, N):
    case = syn.random_case(M, K, N, keep, seed=M + N + 5)
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    say(f"bitmap gauss M={M} K={K} N={N}")
    assert_gates(run(h, case.B16, M), osp.spmm_f64(case.A16, case.mask, case.B16), f"M={M} K={K} N={N}")


@pytest.mark.parametrize("cfg,shape", [(2, 0), (5, 1), (5, 0), (4, 0)])
def test_bitmap_full_size_sampled_rows(cfg, shape):
    case = syn.make_config(cfg, shape)
    say(f"bitmap full {case.name}")
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    rng = np.random.default_rng(9)
    rows = np.array(sorted(set(range(64)) | set(range(case.M - 64, case.M)) |
                           set(rng.choice(case.M, 256, replace=False).tolist())), dtype=np.int64)
    C = run(h, case.B16, case.M)
    assert np.isfinite(C.view(np.float16)).all()
    assert_gates(C[:, rows], osp.spmm_f64(case.A16, case.mask, case.B16, rows=rows), case.name)


def test_bitmap_integer_full_size_cfg2():
    case = syn.make_config(2)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4321, 2, 0])))
    A16 = syn.int_fp16(rng, case.M, case.K)
    B16 = syn.int_fp16(rng, case.N, case.K)
    h = L.lscd_encode_bitmap(A16, case.mask)
    C = run(h, B16, case.M)
    rows = np.arange(0, case.M, 97)
    C64 = osp.spmm_f64(A16, case.mask, B16, rows=rows)
    assert np.array_equal(C[:, rows], osp.fp16_rne(C64))


def test_bitmap_linear_dense_path():
    case = syn.random_case(500, 900, 48, 0.3, seed=23, values="int3")
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    L.lscd_attach_dense(h)
    L.lscd_set_linear_crossover(h, 0)
    B = dev(case.B16)
    C = torch.empty((48, 500), dtype=torch.float16, device="cuda")
    L.lscd_linear(h, B, C)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(np.uint16), osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16)))


def test_bitmap_full_chunk_at_odd_start():
    # A full chunk (8 kept positions) whose run starts at an odd value needs one value past its
    # 16-byte window: lane 5 and lane 62 take it from the next lane, lane 63 from a scalar load.
    # Lane l, chunk g holds row 16*(g//2) + l%16, columns 32*(g%2) + 8*(l//16) .. +7.
    M, K, N = 80, 100, 16
    mask = np.zeros((M, K), dtype=np.uint8)
    mask[0, 0] = 1                      # lane 0, chunk 0: one value, so later runs start odd
    mask[5, 0:8] = 1                    # lane 5, chunk 0: full, start 1
    mask[15, 24:32] = 1                 # lane 63, chunk 0: full, start 9
    mask[32, 32:34] = 1                 # lane 0, chunk 5: two values (chunk 5 starts at 17)
    mask[46, 56:64] = 1                 # lane 62, chunk 5: full, start 19
    mask[47, 56:64] = 1                 # lane 63, chunk 5: full, start 27
    mask[64:, 64:] = 1                  # a ragged, dense second-row tile
    rng = np.random.default_rng(31)
    A16 = syn.int_fp16(rng, M, K)
    B16 = syn.int_fp16(rng, N, K)
    for r, c in ((5, 0), (15, 24), (46, 56), (47, 56)):
        assert ob.lane_bit(r, c)[1] % 8 == 0
    h = L.lscd_encode_bitmap(A16, mask)
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    L.lscd_debug_decode(h, A)
    torch.cuda.synchronize()
    assert np.array_equal(A.cpu().numpy().view(np.uint16), tc.masked(A16, mask))
    assert np.array_equal(run(h, B16, M), osp.fp16_rne(osp.spmm_f64(A16, mask, B16)))


def test_bitmap_linear_path_per_tile_cost():
    # a bitmap handle is costed per tile and per 64-column launch; on this shape (16384 tiles,
    # 80 % sparse) the dispatcher keeps the sparse product for small N, moves to the dense GEMM
    # for large N, and never goes back
    case = syn.random_case(8192, 8192, 1, 0.2, seed=8)
    h = L.lscd_encode_bitmap(case.A16, case.mask)
    L.lscd_attach_dense(h)
    paths = [L.lscd_linear_path(h, N) for N in (1, 16, 32, 64, 65, 128, 200, 256, 512)]
    assert paths[0] == 0 and paths[1] == 0 and paths[-1] == 1, paths
    assert paths == sorted(paths), paths
