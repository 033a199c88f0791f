"""Oracle product C[N][M] = (A*mask) . B^T in fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: Flash-LLM paper review (xllm-io), section 3 "core formulas": the MatMul
is C = A x B with the sparse weight A of shape M x K and the dense feature
matrix B of shape K x N.  Load-as-Sparse / Compute-as-Dense (section 2,
"solution") runs a dense product over the weights once they are unpacked, so
the result is the plain dense product of the decoded A.

Layout reading (the pages leave it open): activations are stored as B[N][K]
(row-major, K contiguous) and the result as C[N][M] -- the layout of
Y = X . W^T for a batch of N token vectors -- i.e. the pages' K x N and M x N
matrices stored column-major.

Arithmetic: every fp16 value converts to fp64 exactly and every product of two
fp16 values is exact in fp64 (22 significant bits); the sums are accumulated
in fp64 by a library matrix product over row blocks, a plain step that does
not reorder anything the definition fixes (a sum's order is free in exact
arithmetic; in fp64 the rounding of sums of at most 2^16 terms of this size is
far below any tolerance used on the result).

Output rounding reading: the GPU result is fp16, rounded once from the fp32
accumulator with round-to-nearest-even.  `fp16_rne` rounds the fp64 oracle the
same way for comparisons that must be bit-exact (integer-valued inputs).
"""
from __future__ import annotations

import numpy as np

_BLOCK_ELEMS = 1 << 23


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact conversion of fp16 bit patterns to fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def spmm_f64(A16: np.ndarray, mask: np.ndarray, B16: np.ndarray, rows=None) -> np.ndarray:
    """C64[n][i] = sum_k A[i][k]*mask[i][k] * B[n][k] for i in `rows` (default: all rows).

    Returns float64 [N][len(rows)].
    """
    M, K = A16.shape
    N, Kb = B16.shape
    if Kb != K:
        raise ValueError("A and B disagree on K")
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    Bt = fp16_to_f64(B16).T                        # [K][N]
    out = np.empty((N, rows.size), dtype=np.float64)
    step = max(1, _BLOCK_ELEMS // max(K, 1))
    for s in range(0, rows.size, step):
        r = rows[s:s + step]
        a = fp16_to_f64(A16[r])
        a[mask[r] == 0] = 0.0
        out[:, s:s + step] = (a @ Bt).T
    return out


def spmm_exact_small(A16: np.ndarray, mask: np.ndarray, B16: np.ndarray):
    """Exact rational result by nested loops (tiny inputs only): list of lists of Fraction."""
    from fractions import Fraction
    M, K = A16.shape
    N = B16.shape[0]
    a = fp16_to_f64(A16)
    b = fp16_to_f64(B16)
    C = [[Fraction(0) for _ in range(M)] for _ in range(N)]
    for n in range(N):
        for i in range(M):
            acc = Fraction(0)
            for k in range(K):
                if mask[i, k]:
                    acc += Fraction(float(a[i, k])) * Fraction(float(b[n, k]))
            C[n][i] = acc
    return C


def fp16_rne(C64: np.ndarray) -> np.ndarray:
    """fp16 bit patterns of C64 rounded to nearest, ties to even (overflow -> inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(C64, dtype=np.float64).astype(np.float16).view(np.uint16)
