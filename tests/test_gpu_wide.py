"""GPU parity of the N > 64 path (wide kernel, launches of <= 256 columns) and of lscd_linear.

* integer-valued inputs: bit-exact against fp16_rne of the oracle for N across the padding
  boundaries (65 .. 520, several launches and a skinny last slice), with forced K splits;
* Gaussian inputs: the tolerance gates (tests/_util.py) on ragged shapes and, with sampled
  rows, at the full OPT-175B MLP2 shape;
* lscd_linear: the dense path (rocBLAS GEMM on the decoded copy) and the sparse path both
  match the oracle; the path follows lscd_set_linear_crossover.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from tests._util import assert_gates, env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L


def run(fn, h, B16, M):
    B = torch.from_numpy(np.ascontiguousarray(B16).view(np.float16)).to("cuda")
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    fn(h, B, C)
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("N", [65, 96, 128, 129, 192, 200, 256, 257, 300, 520])
@pytest.mark.parametrize("splits", [None, "1", "3"])
def test_wide_integer_bit_exact(N, splits):
    case = syn.random_case(333, 1000, N, 0.35, seed=1000 + N, values="int3")
    with env(LSCD_SPLITK=splits):
        h = L.lscd_encode(case.A16, case.mask)
    say(f"wide int N={N} splits_wide={h.info['splits_wide']} Rw={h.info['reg_vectors_wide']}")
    C = run(L.lscd_spmm, h, case.B16, case.M)
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.abs(C64).max() < 2048
    assert np.array_equal(C, osp.fp16_rne(C64))


@pytest.mark.parametrize("M,K,keep", [(64, 64, 0.3), (300, 520, 0.3), (1000, 1111, 0.25), (65, 70, 0.6),
                                      (257, 3000, 0.4), (200, 300, 1.0)])
@pytest.mark.parametrize("N", [80, 128, 256, 384])
def test_wide_gaussian_within_tolerance(M, K, keep, N):
    case = syn.random_case(M, K, N, keep, seed=M + K + N)
    h = L.lscd_encode(case.A16, case.mask)
    say(f"wide gauss M={M} K={K} N={N}")
    C = run(L.lscd_spmm, h, case.B16, M)
    assert_gates(C, osp.spmm_f64(case.A16, case.mask, case.B16), f"M={M} K={K} N={N}")


def test_wide_full_size_sampled_rows():
    case = syn.make_config(4)
    h = L.lscd_encode(case.A16, case.mask)
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set(range(64)) | set(range(case.M - 64, case.M)) |
                           set(rng.choice(case.M, 128, replace=False).tolist())), dtype=np.int64)
    for N in (128, 256):
        B16 = syn.make_config(4, N=N).B16
        say(f"wide full {case.name} N={N} splits_wide={h.info['splits_wide']}")
        C = run(L.lscd_spmm, h, B16, case.M)
        assert np.isfinite(C.view(np.float16)).all()
        assert_gates(C[:, rows], osp.spmm_f64(case.A16, case.mask, B16, rows=rows), f"N={N}")


@pytest.mark.parametrize("N", [16, 100])
def test_tuned_dense_path(N):
    """lscd_tune_dense times hipBLASLt candidates and lscd_linear then runs the fastest; integer
    inputs keep the GEMM bit-exact whichever algorithm (any summation order is exact)."""
    case = syn.random_case(700, 1100, N, 0.3, seed=N + 3, values="int3")
    h = L.lscd_encode(case.A16, case.mask)
    B = torch.from_numpy(case.B16.view(np.float16)).to("cuda")
    C = torch.empty((N, case.M), dtype=torch.float16, device="cuda")
    with pytest.raises(L.LSCDError):
        L.lscd_tune_dense(h, B, C)                              # no dense copy yet
    L.lscd_attach_dense(h)
    ts0, td0, measured0 = L.lscd_linear_times(h, N)
    assert not measured0
    assert (ts0, td0) == L.lscd_linear_model(case.M, case.K, h.info["nnz_padded"], h.info["num_tiles"], N)
    us, n = L.lscd_tune_dense(h, B, C)
    ts, td, measured = L.lscd_linear_times(h, N)
    say(f"tuned dense N={N}: {us:.1f} us over {n} candidates; sparse {ts:.1f} us")
    assert n >= 1 and us > 0 and measured and td == us and ts > 0
    assert L.lscd_linear_path(h, N) == (1 if us < ts else 0)     # the two measured times decide
    L.lscd_set_linear_crossover(h, 0)
    want = osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16))
    assert np.array_equal(run(L.lscd_linear, h, case.B16, case.M), want)


def test_linear_paths():
    case = syn.random_case(500, 900, 96, 0.3, seed=21, values="int3")
    h = L.lscd_encode(case.A16, case.mask)
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    want = osp.fp16_rne(C64)
    assert L.lscd_linear_path(h, 96) == 0                       # no dense copy yet: sparse
    assert np.array_equal(run(L.lscd_linear, h, case.B16, case.M), want)
    L.lscd_attach_dense(h)
    L.lscd_attach_dense(h)                                      # idempotent
    L.lscd_set_linear_crossover(h, 0)                           # always dense
    assert L.lscd_linear_path(h, 96) == 1
    say("linear dense path")
    # integer inputs: fp32 accumulation is exact in any order, so the GEMM is bit-exact too
    assert np.array_equal(run(L.lscd_linear, h, case.B16, case.M), want)
    L.lscd_set_linear_crossover(h, 1 << 20)                     # always sparse
    assert L.lscd_linear_path(h, 96) == 0
    assert np.array_equal(run(L.lscd_linear, h, case.B16, case.M), want)
    L.lscd_set_linear_crossover(h, -1)                          # back to the cost model
    g = syn.random_case(500, 900, 300, 0.3, seed=22)
    hg = L.lscd_encode(g.A16, g.mask)
    L.lscd_attach_dense(hg)
    for N, cross in ((300, 0), (300, 1 << 20), (16, 0)):
        L.lscd_set_linear_crossover(hg, cross)
        B16 = g.B16[:N]
        say(f"linear gauss N={N} path={L.lscd_linear_path(hg, N)}")
        assert_gates(run(L.lscd_linear, hg, B16, g.M), osp.spmm_f64(g.A16, g.mask, B16), f"linear N={N}")


def test_wide_limits():
    case = syn.random_case(130, 200, 8, 0.3, seed=13)
    h = L.lscd_encode(case.A16, case.mask)
    B = torch.zeros((1, 200), dtype=torch.float16, device="cuda")
    C = torch.zeros((1, 130), dtype=torch.float16, device="cuda")
    st = L._lib.lscd_spmm(L.ctypes.c_void_p(h.ptr), L.ctypes.c_void_p(B.data_ptr()),
                          L.ctypes.c_void_p(C.data_ptr()), L.LSCD_MAX_N + 1, None)
    assert st == L.LSCD_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()


def test_split_plan_192_row_blocks():
    """192 row blocks of 64 rows at 50 % sparsity on 256 CUs: the N > 64 kernel takes 4 splits
    (768 workgroups, three per CU: the resident slots, and the most the planner allows), the
    shared-B launch at N = 64 fills its slots.  The product at N = 128 with this plan is
    bit-exact on integer inputs (sampled rows)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([31337, 128])))
    M, K, N = 12288, 2048, 128
    A16 = syn.int_fp16(rng, M, K)
    mask = (rng.random((M, K), dtype=np.float32) < 0.5).astype(np.uint8)
    h = L.lscd_encode(A16, mask)
    info = h.info
    say(f"plan cus={cus} tile={info['tile_m']} S={info['splits']} Sw={info['splits_wide']} variant={info['variant']}")
    if cus == 256:
        assert info["tile_m"] == 64
        assert info["splits_wide"][0] == 4
        # N = 64 fills the resident slots: groups of three row blocks x 8 splits (512), or of
        # four x 10 (480) where the three-wavefront kernel has no instantiation for the stage
        assert (info["variant"][2], info["splits"][2]) in ((6, 8), (0, 10))
    B16 = syn.int_fp16(rng, N, K)
    B = torch.from_numpy(B16.view(np.float16)).to("cuda")
    C = torch.full((N, M), float("nan"), dtype=torch.float16, device="cuda")
    L.lscd_spmm(h, B, C)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(64)) | set(range(M - 64, M)) |
                           set(rng.choice(M, size=256, replace=False).tolist())), dtype=np.int64)
    C64 = osp.spmm_f64(A16, mask, B16, rows=rows)
    assert np.abs(C64).max() < 65504
    assert np.array_equal(C.cpu().numpy().view(np.uint16)[:, rows], osp.fp16_rne(C64))


def _inflate(words, offs, reps):
    """Every tile's words repeated `reps` times: duplicates with the same bits are valid padding
    (a word placed twice lands on the same position with the same value)."""
    w2, o2 = [], [0]
    for t in range(len(offs) - 1):
        tile = words[offs[t]:offs[t + 1]]
        w2.append(np.tile(tile, reps))
        o2.append(o2[-1] + reps * len(tile))
    return np.concatenate(w2).astype(np.uint32), np.array(o2, dtype=np.uint32)


@pytest.mark.parametrize("tm", [64, 128])
@pytest.mark.parametrize("N", [16, 64, 128, 256])
def test_words_past_every_register_stage(tm, N):
    """Dense tiles whose words are repeated so that a tile holds more words than any register
    stage (64-row tiles: 8192 words; 128-row tiles: 16384 words): the tail loops of the skinny
    and N > 64 kernels place the rest, and the integer product stays bit-exact."""
    case = syn.random_case(200, 150, N, 1.0, seed=77 + tm + N, values="int3")
    w, o = L.lscd_pack(case.A16, case.mask, tm, 64)
    w2, o2 = _inflate(w, o, 2)
    assert int(np.diff(o2).max()) > 4 * 256 * (4 if tm == 64 else 8)
    h = L.lscd_import(w2, o2, case.M, case.K, tm, 64)
    say(f"inflated tm={tm} N={N} max_tile_words={h.info['max_tile_words']} variant={h.info['variant']} "
        f"Rw={h.info['reg_vectors_wide']}")
    C = run(L.lscd_spmm, h, case.B16, case.M)
    assert np.array_equal(C, osp.fp16_rne(osp.spmm_f64(case.A16, case.mask, case.B16)))
