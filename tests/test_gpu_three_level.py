"""GPU parity of the three-level path (lscd_encode_three_level + lscd_spmm / lscd_debug_decode).

Bit-exact: the decoded matrix and the exported blob against the oracle encoder (dense tiles,
whose excess entries all go to the residual words, included), integer-valued products for N
across the 16 / 32 / 64-column launch boundaries with forced K splits, at small shapes and at
a full OPT shape.  Tolerance gates (tests/_util.py) for Gaussian inputs on ragged shapes and,
with sampled rows, at full OPT shapes at 50% and 60% sparsity.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from oracle import three_level as otl
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


SHAPES = [(64, 64, 0.5), (256, 256, 0.45), (300, 520, 0.5), (1000, 1111, 0.4), (1, 1, 1.0), (65, 70, 0.6),
          (512, 4096, 0.5), (257, 3000, 0.55), (200, 300, 1.0), (100, 300, 0.0), (130, 200, 0.1)]


@pytest.mark.parametrize("M,K,keep", SHAPES)
def test_three_level_decode_and_export_bit_exact(M, K, keep):
    case = syn.random_case(M, K, 1, keep, seed=M * 7 + K)
    say(f"three-level decode M={M} K={K} keep={keep}")
    h = L.lscd_encode_three_level(case.A16, case.mask)
    assert h.info["format"] == 2 and h.info["nnz"] == int(case.mask.sum()) and h.info["reg_vectors"] == 0
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    L.lscd_debug_decode(h, A)
    torch.cuda.synchronize()
    assert np.array_equal(A.cpu().numpy().view(np.uint16), tc.masked(case.A16, case.mask))
    words, offs = L.lscd_export(h)
    ow, oo = otl.encode(case.A16, case.mask)
    assert np.array_equal(words, ow) and np.array_equal(offs, oo)


@pytest.mark.parametrize("N", [1, 8, 16, 17, 32, 33, 48, 64, 65, 100])
@pytest.mark.parametrize("splits", [None, "1", "3"])
def test_three_level_integer_bit_exact(N, splits):
    case = syn.random_case(333, 1000 + 8 * N, N, 0.5, seed=N + 91, values="int3")
    with env(LSCD_SPLITK=splits):
        h = L.lscd_encode_three_level(case.A16, case.mask)
    say(f"three-level int N={N} S={h.info['splits']}")
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.abs(C64).max() < 2048
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(C64))


@pytest.mark.parametrize("keep", [1.0, 0.75, 0.05])
def test_three_level_integer_dense_and_sparse_tiles(keep):
    """Dense tiles (every excess entry in the residual words, more than 64 units per tile) and
    nearly empty ones (dummy points across long gaps)."""
    case = syn.random_case(200, 650, 24, keep, seed=5, values="int3")
    h = L.lscd_encode_three_level(case.A16, case.mask)
    say(f"three-level int keep={keep}")
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.array_equal(run(h, case.B16, case.M), osp.fp16_rne(C64))


@pytest.mark.parametrize("M,K,keep", SHAPES[:8])
@pytest.mark.parametrize("N", [8, 16, 32, 64])
def test_three_level_gaussian_within_tolerance(M, K, keep, N):
    case = syn.random_case(M, K, N, keep, seed=M + N + 11)
    h = L.lscd_encode_three_level(case.A16, case.mask)
    say(f"three-level gauss M={M} K={K} N={N}")
    assert_gates(run(h, case.B16, M), osp.spmm_f64(case.A16, case.mask, case.B16), f"M={M} K={K} N={N}")


@pytest.mark.parametrize("cfg,shape,N,sparsity", [(5, 1, 16, None), (5, 0, 64, None), (5, 3, 32, None),
                                                  (4, 0, 64, None), (5, 1, 8, 0.6)])
def test_three_level_full_size_sampled_rows(cfg, shape, N, sparsity):
    case = syn.make_config(cfg, shape, N=N, sparsity=sparsity)
    say(f"three-level full {case.name}")
    h = L.lscd_encode_three_level(case.A16, case.mask)
    rng = np.random.default_rng(13)
    rows = np.array(sorted(set(range(64)) | set(range(case.M - 64, case.M)) |
                           set(rng.choice(case.M, 256, replace=False).tolist())), dtype=np.int64)
    C = run(h, case.B16, case.M)
    assert np.isfinite(C.view(np.float16)).all()
    assert_gates(C[:, rows], osp.spmm_f64(case.A16, case.mask, case.B16, rows=rows), case.name)


def test_three_level_integer_full_size_outproj():
    case = syn.make_config(5, 1, N=64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4321, 5, 1])))
    A16 = syn.int_fp16(rng, case.M, case.K)
    B16 = syn.int_fp16(rng, case.N, case.K)
    h = L.lscd_encode_three_level(A16, case.mask)
    C = run(h, B16, case.M)
    rows = np.arange(0, case.M, 97)
    C64 = osp.spmm_f64(A16, case.mask, B16, rows=rows)
    assert np.array_equal(C[:, rows], osp.fp16_rne(C64))


def test_three_level_run_to_run_identical():
    case = syn.random_case(700, 2000, 32, 0.5, seed=3)
    h = L.lscd_encode_three_level(case.A16, case.mask)
    assert np.array_equal(run(h, case.B16, case.M), run(h, case.B16, case.M))


def test_three_level_linear_dense_path():
    case = syn.random_case(500, 900, 48, 0.5, seed=29, values="int3")
    h = L.lscd_encode_three_level(case.A16, case.mask)
    L.lscd_attach_dense(h)
    L.lscd_set_linear_crossover(h, 0)
    B = dev(case.B16)
    C = torch.empty((48, 500), dtype=torch.float16, device="cuda")
    L.lscd_linear(h, B, C)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(np.uint16), osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16)))
