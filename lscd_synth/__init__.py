"""Seeded synthetic inputs for the sparse x skinny matrix product.

This module only draws numbers: pruned fp16 weight matrices A[M][K] with their
keep masks, and dense fp16 activations B[N][K].  It holds none of the product's
arithmetic, so both the CPU oracle's tests and the GPU path's tests and
benchmark can take their inputs from here without sharing any code of the
method itself.

Workload shapes follow the skinny MatMuls of an OPT decoder layer (QKV
projection, output projection, MLP1, MLP2; M is the output dimension, K the
input dimension, N the batch of tokens in a decode step), as laid out in the
Flash-LLM paper review (xllm-io), section 3 "overall framework", table of the
four skinny MatMuls.  The sparsity levels and the OPT hidden sizes are those of
the five benchmark configurations listed in `CONFIGS` below.  No checkpoint or
dataset is used: values are drawn, not loaded.

Random streams: `numpy.random.Generator(PCG64(SeedSequence([seed, cfg, role,
shape])))`, role 0 = A values, 1 = mask, 2 = B.  Draws are taken in float32
and rounded to fp16 with round-to-nearest-even (`astype(np.float16)`).  Large
matrices are drawn in blocks of whole rows from the one stream, in row order,
so the result does not depend on memory limits of the machine.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ROLE_A, ROLE_MASK, ROLE_B = 0, 1, 2
DEFAULT_SEED = 1234
SIGMA_A = 0.02          # weight scale: N(0, 0.02), the OPT init convention
SIGMA_B = 1.0           # activations: N(0, 1)
_CHUNK_ELEMS = 1 << 24  # elements per drawn block (rows are never split)


@dataclasses.dataclass
class Case:
    """One seeded problem instance: C[N][M] = (A*mask)[M][K] . B[N][K]^T."""
    name: str
    M: int
    K: int
    N: int
    A16: np.ndarray     # uint16 [M][K], fp16 bit patterns of the weights
    mask: np.ndarray    # uint8  [M][K], 1 = keep
    B16: np.ndarray     # uint16 [N][K], fp16 bit patterns of the activations

    @property
    def nnz(self) -> int:
        return int(np.count_nonzero(self.mask))

    @property
    def sparsity(self) -> float:
        return 1.0 - self.nnz / float(self.M * self.K)


def _rng(seed: int, cfg: int, role: int, shape: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, role, shape])))


def _row_blocks(M: int, K: int):
    rows = max(1, _CHUNK_ELEMS // max(K, 1))
    for r0 in range(0, M, rows):
        yield r0, min(M, r0 + rows)


def gaussian_fp16(rng: np.random.Generator, rows: int, cols: int, sigma: float) -> np.ndarray:
    """fp16 bit patterns of sigma * N(0,1) draws (float32, then RNE to fp16)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0, r1 in _row_blocks(rows, cols):
        x = rng.standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        x *= np.float32(sigma)
        out[r0:r1] = x.astype(np.float16).view(np.uint16)
    return out


def int_fp16(rng: np.random.Generator, rows: int, cols: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """fp16 bit patterns of integers drawn uniformly from [lo, hi] (exact in fp16)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0, r1 in _row_blocks(rows, cols):
        x = rng.integers(lo, hi + 1, size=(r1 - r0, cols), dtype=np.int8)
        out[r0:r1] = x.astype(np.float16).view(np.uint16)
    return out


def bernoulli_mask(rng: np.random.Generator, rows: int, cols: int, keep: float) -> np.ndarray:
    """i.i.d. keep mask: each position kept with probability `keep`."""
    out = np.empty((rows, cols), dtype=np.uint8)
    for r0, r1 in _row_blocks(rows, cols):
        out[r0:r1] = rng.random(size=(r1 - r0, cols), dtype=np.float32) < np.float32(keep)
    return out


def row_varied_mask(rng: np.random.Generator, rows: int, cols: int, keep: float, spread: float) -> np.ndarray:
    """Keep mask whose per-row keep probability varies by up to +-spread (relative).

    Row i keeps each position with probability keep*(1+u_i), u_i ~ U[-spread, spread],
    drawn first (one per row) from the same stream as the Bernoulli draws.
    """
    p = (keep * (1.0 + rng.uniform(-spread, spread, size=rows))).astype(np.float32)
    out = np.empty((rows, cols), dtype=np.uint8)
    for r0, r1 in _row_blocks(rows, cols):
        out[r0:r1] = rng.random(size=(r1 - r0, cols), dtype=np.float32) < p[r0:r1, None]
    return out


def topk_magnitude_mask(A16: np.ndarray, k: int) -> np.ndarray:
    """Keep exactly the k largest |value| per row (magnitude pruning); ties go to the lower column.

    For finite fp16, ordering of |x| equals ordering of the bit pattern with the
    sign bit cleared, so the selection is done on integers.
    """
    M, K = A16.shape
    k = int(k)
    out = np.zeros((M, K), dtype=np.uint8)
    if k <= 0:
        return out
    if k >= K:
        out[:] = 1
        return out
    for r0, r1 in _row_blocks(M, K):
        mag = (A16[r0:r1] & np.uint16(0x7FFF)).astype(np.int32)
        kth = np.partition(mag, K - k, axis=1)[:, K - k]          # k-th largest per row
        gt = mag > kth[:, None]
        need = k - gt.sum(axis=1)                                    # how many ties to take
        eq = mag == kth[:, None]
        take_eq = eq & (np.cumsum(eq, axis=1, dtype=np.int32) <= need[:, None])
        out[r0:r1] = gt | take_eq
    return out


# --------------------------------------------------------------------------------------
# The five benchmark configurations (OPT-shaped skinny MatMuls).
# --------------------------------------------------------------------------------------

#: config id -> list of (shape name, M, K); N and sparsity below.
SHAPES = {
    1: [("tiny", 1024, 1024)],
    2: [("opt30b_mlp1", 28672, 7168)],
    3: [("opt66b_qkv", 27648, 9216)],
    4: [("opt175b_mlp2", 12288, 49152)],
    5: [("opt175b_qkv", 36864, 12288), ("opt175b_outproj", 12288, 12288),
        ("opt175b_mlp1", 49152, 12288), ("opt175b_mlp2", 12288, 49152)],
}
DEFAULT_N = {1: 8, 2: 16, 3: 32, 4: 64, 5: 16}
SPARSITY = {1: 0.8, 2: 0.8, 3: 0.7, 4: 0.6, 5: 0.5}
CONFIGS = {
    1: "tiny 1024x1024, N=8, 80% i.i.d. Bernoulli",
    2: "OPT-30B MLP1 28672x7168, N=16, 80% with +-20% per-row keep variation",
    3: "OPT-66B QKV 27648x9216, N=32, 70% magnitude-pruned (top-30% |w| per row)",
    4: "OPT-175B MLP2 12288x49152, N=64, 60% i.i.d. Bernoulli",
    5: "OPT-175B layer sweep (QKV/OutProj/MLP1/MLP2) at 50% i.i.d., N in {8,16,32,64}",
}


def make_config(cfg: int, shape: int = 0, N: Optional[int] = None, sparsity: Optional[float] = None,
                seed: int = DEFAULT_SEED, rows: Optional[int] = None) -> Case:
    """Build configuration `cfg` (1..5), shape index `shape` (config 5 has four).

    `N` overrides the batch width (config 5 sweeps it), `sparsity` overrides the
    prune level (e.g. config 5 shapes re-run at 60%), `rows` keeps only the first
    `rows` rows (same draws as the full matrix for those rows, for quick tests).
    """
    name, M, K = SHAPES[cfg][shape]
    N = DEFAULT_N[cfg] if N is None else int(N)
    beta = SPARSITY[cfg] if sparsity is None else float(sparsity)
    keep = 1.0 - beta
    Mg = M if rows is None else min(M, int(rows))
    A16 = gaussian_fp16(_rng(seed, cfg, ROLE_A, shape), Mg, K, SIGMA_A)
    mrng = _rng(seed, cfg, ROLE_MASK, shape)
    if cfg == 2 and sparsity is None:
        if rows is None:
            mask = row_varied_mask(mrng, M, K, keep, 0.2)
        else:
            # draw the per-row probabilities for all M rows so row i is the same as in the full matrix
            p = (keep * (1.0 + mrng.uniform(-0.2, 0.2, size=M))).astype(np.float32)
            mask = np.empty((Mg, K), dtype=np.uint8)
            for r0, r1 in _row_blocks(Mg, K):
                mask[r0:r1] = mrng.random(size=(r1 - r0, K), dtype=np.float32) < p[r0:r1, None]
    elif cfg == 3 and sparsity is None:
        mask = topk_magnitude_mask(A16, int(round(keep * K)))
    else:
        mask = bernoulli_mask(mrng, Mg, K, keep)
    B16 = gaussian_fp16(_rng(seed, cfg, ROLE_B, shape), N, K, SIGMA_B)
    label = f"cfg{cfg}_{name}_N{N}_s{int(round(beta * 100))}"
    return Case(label, Mg, K, N, A16, mask, B16)


def random_case(M: int, K: int, N: int, keep: float, seed: int = 7, values: str = "gauss",
                name: str = "random") -> Case:
    """Small seeded case for unit tests.

    values: "gauss" (A ~ N(0,0.02), B ~ N(0,1)), "int3" (A, B integers in [-3,3],
    exact in fp16 and with every partial sum exact in fp32 for K < 2^20),
    "unit" (A ~ N(0,1) too).
    """
    ra, rm, rb = (_rng(seed, 99, role, M * 131 + K * 7 + N) for role in (ROLE_A, ROLE_MASK, ROLE_B))
    if values == "int3":
        A16 = int_fp16(ra, M, K)
        B16 = int_fp16(rb, N, K)
    elif values == "unit":
        A16 = gaussian_fp16(ra, M, K, 1.0)
        B16 = gaussian_fp16(rb, N, K, 1.0)
    else:
        A16 = gaussian_fp16(ra, M, K, SIGMA_A)
        B16 = gaussian_fp16(rb, N, K, SIGMA_B)
    mask = bernoulli_mask(rm, M, K, keep)
    return Case(name, M, K, N, A16, mask, B16)


def identity_B(K: int, cols) -> np.ndarray:
    """B16 with B[n][cols[n]] = 1.0 and zero elsewhere (selects columns of A)."""
    B = np.zeros((len(cols), K), dtype=np.uint16)
    for n, c in enumerate(cols):
        B[n, c] = 0x3C00
    return B
