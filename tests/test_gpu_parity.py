"""GPU parity of the HIP path against the CPU oracle, through the C ABI (small and ragged sizes).

Bit-exact: the decoded matrix (lscd_debug_decode), integer-valued products, identity-B
column selection, run-to-run repeats and within-tile shuffles.  Tolerance (MAX_REL /
FRO_REL in tests/_util.py) for Gaussian inputs.  Split-K is exercised with forced splits.
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


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).to("cuda")


def host(t):
    return t.detach().cpu().numpy().view(np.uint16)


def run_spmm(h, B16, M):
    B = dev(B16)
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    L.lscd_spmm(h, B, C)
    torch.cuda.synchronize()
    return host(C)


SHAPES = [  # (M, K, keep) -- several tiles and ragged tails in M and K
    (64, 64, 0.3), (256, 256, 0.2), (300, 520, 0.3), (1000, 1111, 0.25), (129, 8 * 97, 0.5),
    (1, 1, 1.0), (65, 70, 0.6), (512, 4096, 0.1), (257, 3000, 0.4),
]


@pytest.mark.parametrize("M,K,keep", SHAPES)
def test_decode_bit_exact(M, K, keep):
    say(f"decode M={M} K={K} keep={keep}")
    case = syn.random_case(M, K, 1, keep, seed=M * 7 + K)
    h = L.lscd_encode(case.A16, case.mask)
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    L.lscd_debug_decode(h, A)
    torch.cuda.synchronize()
    assert np.array_equal(host(A), tc.masked(case.A16, case.mask))


def test_decode_dense_and_overflow_paths():
    """A dense tile (4096 words) and tiles larger than the register stage (forced small stage)."""
    case = syn.random_case(200, 300, 1, 1.0, seed=2)
    for cap in (None, "2"):
        with env(LSCD_MAX_R=cap):
            h = L.lscd_encode(case.A16, case.mask)
        say(f"decode dense R={h.info['reg_vectors']}")
        A = torch.empty((200, 300), dtype=torch.float16, device="cuda")
        L.lscd_debug_decode(h, A)
        torch.cuda.synchronize()
        assert np.array_equal(host(A), tc.masked(case.A16, case.mask))


@pytest.mark.parametrize("N", [1, 7, 8, 16, 17, 32, 33, 48, 64])
@pytest.mark.parametrize("splits", [None, "1", "3"])
@pytest.mark.parametrize("variant", ["indep", "shared", "shared3"])
def test_integer_bit_exact(N, splits, variant):
    """Integer inputs: every partial sum is exact in fp32, so C must equal fp16_rne(C_oracle) bit for bit.

    Runs the product kernel variants: the independent-wavefront one exists for N <= 32; above
    that the shared-B kernel runs, with four row blocks per workgroup ("indep", "shared") or
    three ("shared3"; at N <= 32 that setting leaves the default kernel).
    """
    case = syn.random_case(333, 1000 + 8 * N, N, 0.35, seed=N, values="int3")
    with env(LSCD_SPLITK=splits, LSCD_KERNEL=variant):
        h = L.lscd_encode(case.A16, case.mask)
    say(f"int N={N} S={h.info['splits'][L.npad_index(N)]} variant={h.info['variant'][L.npad_index(N)]}")
    C = run_spmm(h, case.B16, case.M)
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    assert np.abs(C64).max() < 2048
    assert np.array_equal(C, osp.fp16_rne(C64))


@pytest.mark.parametrize("M,K,keep", SHAPES)
@pytest.mark.parametrize("N", [8, 16, 32, 64])
@pytest.mark.parametrize("variant", ["indep", "shared", "shared3"])
def test_gaussian_within_tolerance(M, K, keep, N, variant):
    case = syn.random_case(M, K, N, keep, seed=M + N)
    with env(LSCD_KERNEL=variant):
        h = L.lscd_encode(case.A16, case.mask)
    say(f"gauss M={M} K={K} N={N} S={h.info['splits'][L.npad_index(N)]} R={h.info['reg_vectors']}")
    C = run_spmm(h, case.B16, M)
    assert_gates(C, osp.spmm_f64(case.A16, case.mask, case.B16), f"M={M} K={K} N={N}")


def test_identity_b_selects_columns():
    case = syn.random_case(700, 900, 1, 0.3, seed=4)
    cols = [0, 899, 64, 63, 128, 450, 451, 800, 5, 5, 77, 640, 641, 700, 1, 2]
    B16 = syn.identity_B(case.K, cols)
    for splits in (None, "1"):
        with env(LSCD_SPLITK=splits):
            h = L.lscd_encode(case.A16, case.mask)
        C = run_spmm(h, B16, case.M)
        Am = tc.masked(case.A16, case.mask)
        for n, c in enumerate(cols):
            want = Am[:, c].copy()
            want[want == 0x8000] = 0      # -0 * 1 + (+0 * x) sums to +0
            assert np.array_equal(C[n], want), (n, c)


def test_deterministic_and_split_independent_within_tolerance():
    case = syn.random_case(1024, 2048, 32, 0.25, seed=11)
    C64 = osp.spmm_f64(case.A16, case.mask, case.B16)
    results = {}
    for splits in ("1", "2", "5"):
        with env(LSCD_SPLITK=splits):
            h = L.lscd_encode(case.A16, case.mask)
        a = run_spmm(h, case.B16, case.M)
        b = run_spmm(h, case.B16, case.M)
        assert np.array_equal(a, b)                 # bit-reproducible run to run
        assert_gates(a, C64, f"S={splits}")
        results[splits] = a


def test_shuffled_tiles_give_identical_result():
    case = syn.random_case(400, 700, 16, 0.3, seed=12)
    h = L.lscd_encode(case.A16, case.mask)
    ref = run_spmm(h, case.B16, case.M)
    words, offs = L.lscd_export(h)
    rng = np.random.default_rng(0)
    w2 = words.copy()
    for t in range(offs.size - 1):
        rng.shuffle(w2[offs[t]:offs[t + 1]])
    h2 = L.lscd_import(w2, offs, case.M, case.K)
    assert np.array_equal(run_spmm(h2, case.B16, case.M), ref)
    # export round trip equals the host encoder's output
    pw, po = L.lscd_pack(case.A16, case.mask)
    assert np.array_equal(words, pw) and np.array_equal(offs, po)


def test_edge_cases():
    case = syn.random_case(130, 200, 16, 0.3, seed=13)
    h = L.lscd_encode(case.A16, case.mask)
    B = dev(case.B16)
    C = torch.zeros((16, 130), dtype=torch.float16, device="cuda")
    # N = 0 is a no-op success
    assert L._lib.lscd_spmm(L.ctypes.c_void_p(h.ptr), L.ctypes.c_void_p(B.data_ptr()),
                            L.ctypes.c_void_p(C.data_ptr()), 0, None) == L.LSCD_SUCCESS
    # N above LSCD_MAX_N not supported; misaligned pointers rejected
    assert L._lib.lscd_spmm(L.ctypes.c_void_p(h.ptr), L.ctypes.c_void_p(B.data_ptr()),
                            L.ctypes.c_void_p(C.data_ptr()), L.LSCD_MAX_N + 1, None) == L.LSCD_ERROR_NOT_SUPPORTED
    assert L._lib.lscd_spmm(L.ctypes.c_void_p(h.ptr), L.ctypes.c_void_p(B.data_ptr() + 2),
                            L.ctypes.c_void_p(C.data_ptr()), 16, None) == L.LSCD_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert not C.any()
    # fully pruned matrix: exact +0.0 everywhere
    z = syn.random_case(100, 300, 8, 0.0, seed=1)
    hz = L.lscd_encode(z.A16, z.mask)
    assert hz.info["nnz"] == 0
    assert np.array_equal(run_spmm(hz, z.B16, 100), np.zeros((8, 100), np.uint16))
    # a tile format the kernel is not built for is refused by the product (but packs and imports)
    ht = L.lscd_encode_tiled(case.A16, case.mask, 32, 128)
    with pytest.raises(L.LSCDError) as ei:
        L.lscd_spmm(ht, B, C)
    assert ei.value.status == L.LSCD_ERROR_NOT_SUPPORTED


def test_allocation_failure_is_a_status():
    """The allocation-failure hook makes handle creation report OUT_OF_MEMORY (nothing is left
    allocated: the sanitizer build of the host code checks the same path for leaks), and a
    later encode succeeds."""
    case = syn.random_case(130, 200, 8, 0.3, seed=15)
    for enc in (L.lscd_encode, L.lscd_encode_bitmap, L.lscd_encode_three_level):
        with env(LSCD_TEST_FAIL_ALLOC="1"):
            with pytest.raises(L.LSCDError) as ei:
                enc(case.A16, case.mask)
        assert ei.value.status == L.LSCD_ERROR_OUT_OF_MEMORY
    h = L.lscd_encode(case.A16, case.mask)
    assert_gates(run_spmm(h, case.B16, 130), osp.spmm_f64(case.A16, case.mask, case.B16), "after the failures")


def test_other_stream_and_graph_replay():
    case = syn.random_case(900, 1500, 24, 0.3, seed=14)
    h = L.lscd_encode(case.A16, case.mask)
    B = dev(case.B16)
    ref = run_spmm(h, case.B16, case.M)
    s = torch.cuda.Stream()
    C = torch.empty((24, 900), dtype=torch.float16, device="cuda")
    with torch.cuda.stream(s):
        L.lscd_spmm(h, B, C)
    s.synchronize()
    assert np.array_equal(host(C), ref)
    # captured into a HIP graph and replayed, with eager work between replays
    g = torch.cuda.CUDAGraph()
    Cg = torch.empty_like(C)
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        with torch.cuda.graph(g, stream=s2):
            L.lscd_spmm(h, B, Cg)
    for i in range(4):
        Cg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Cg), ref), i
        run_spmm(h, case.B16, case.M)


def test_single_hip_runtime_loaded():
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs
