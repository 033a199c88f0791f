"""GPU parity for every register-stage size of the Tiled-CSL product kernels.

The host picks R, the 128-bit staging vectors per lane, from the largest tile: a tile of w
words needs ceil(w / 256) vectors, rounded up to an instantiated size ({2 .. 12, 16} for 64-row
tiles, {4, 6 .. 12} for taller ones).  Each size is its own kernel instantiation, so each runs
here once, on a matrix built to need exactly that size:
  * per-tile nonzero counts drawn from ((R - 1) * 256, R * 256] (from 1 for R = 2), one tile at
    the top of the range (with a count that is not a multiple of 4, so the tile ends in padding
    words), one empty tile;
  * ragged M and K (the last row block and k tile are partial; K stays a multiple of 8);
  * every kernel variant the tile height has at N padded to 16, 32 and 64, the wide kernel at
    N = 128, with the planned and with forced K splits;
  * integer values: C must equal fp16_rne of the fp64 oracle bit for bit.
"""
import numpy as np
import pytest

import lscd_synth as syn
from oracle import spmm as osp
from tests._util import env, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import unstructured_sparse_skinny_amd as L

# kernel kinds reported in lscd_info_t.variant
SHARED, INDEP, INDEP8, WIDE, SHARED3 = 0, 1, 2, 3, 6

STAGES_64 = [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 16]
STAGES_TALL = [4, 6, 7, 8, 9, 10, 11, 12]
HEIGHTS = [80, 96, 112, 128]


def shared3_expected(R, tm):
    """Stage sizes with a three-row-block shared-B instantiation (two workgroups per CU)."""
    rg = tm // 16
    if rg == 4:
        return R not in (8, 16)
    if rg == 5:
        return R <= 10
    if rg <= 7:
        return R <= 8
    return R <= 6


def stage_case(tm, R, seed):
    """Integer case whose 64-column tiles of tm rows need exactly R staging vectors."""
    MB, KT = 7, 5
    M, K = tm * MB - 5, 64 * KT - 24
    base = syn.random_case(M, K, 128, 1.0, seed=seed, values="int3")
    rng = np.random.default_rng(seed)
    lo, hi = (R - 1) * 256 + 1, R * 256
    if R == 2:
        lo = 1
    mask = np.zeros((M, K), dtype=bool)
    for rb in range(MB):
        r0, r1 = rb * tm, min(M, rb * tm + tm)
        for kt in range(KT):
            c0, c1 = kt * 64, min(K, kt * 64 + 64)
            npos = (r1 - r0) * (c1 - c0)
            if (rb, kt) == (0, 1):
                n = 0                                   # an empty tile
            elif (rb, kt) == (1, 2):
                n = hi - 3                              # the largest tile, ending in padding
            else:
                n = int(rng.integers(lo, hi + 1))
            n = min(n, npos)
            pos = rng.choice(npos, size=n, replace=False)
            sub = np.zeros(npos, dtype=bool)
            sub[pos] = True
            mask[r0:r1, c0:c1] = sub.reshape(r1 - r0, c1 - c0)
    return base.A16, mask, base.B16


def run(h, B16, M):
    B = torch.from_numpy(np.ascontiguousarray(B16).view(np.float16)).to("cuda")
    C = torch.full((B16.shape[0], M), float("nan"), dtype=torch.float16, device="cuda")
    L.lscd_spmm(h, B, C)
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint16)


def check_all_variants(tm, R):
    A16, mask, B128 = stage_case(tm, R, seed=1000 * tm + R)
    M, K = A16.shape
    words, offs = L.lscd_pack(A16, mask, tm, 64)
    assert int(np.diff(offs).max()) == R * 256
    tall = tm != 64
    runs = []
    for N in (13, 32, 50, 128):
        npad = 16 if N <= 16 else (32 if N <= 32 else (64 if N <= 64 else 128))
        if npad <= 32:
            kinds = [(None, INDEP8)] if tall else [("indep", INDEP), ("indep8", INDEP8), ("shared", SHARED)]
        elif npad == 64:
            kinds = [("shared", SHARED), ("shared3", SHARED3 if shared3_expected(R, tm) else SHARED)]
        else:
            kinds = [(None, WIDE)]
        for kernel, kind in kinds:
            runs.append((N, npad, kernel, kind))
    C64 = {N: osp.spmm_f64(A16, mask, B128[:N]) for N in (13, 32, 50, 128)}
    for N, npad, kernel, kind in runs:
        want = osp.fp16_rne(C64[N])
        assert np.abs(C64[N]).max() < 2048
        for splits in (None, "3"):
            with env(LSCD_KERNEL=kernel, LSCD_SPLITK=splits):
                h = L.lscd_import(words, offs, M, K, tm, 64)
            info = h.info
            assert info["reg_vectors"] == R, (info["reg_vectors"], R)
            if npad <= 64:
                got_kind = info["variant"][L.npad_index(N)]
                S = info["splits"][L.npad_index(N)]
            else:
                got_kind, S = WIDE, info["splits_wide"][0]
            say(f"stage tm={tm} R={R} N={N} kernel={kernel} kind={got_kind} S={S} splits={splits} "
                f"Rw={info['reg_vectors_wide']}")
            assert got_kind == kind, (got_kind, kind)
            if splits == "3":
                assert S == 3
            assert np.array_equal(run(h, B128[:N], M), want), (tm, R, N, kernel, splits)


@pytest.mark.parametrize("R", STAGES_64)
def test_every_stage_64_row_tiles(R):
    check_all_variants(64, R)


@pytest.mark.parametrize("R", STAGES_TALL)
@pytest.mark.parametrize("tm", HEIGHTS)
def test_every_stage_tall_tiles(tm, R):
    check_all_variants(tm, R)
