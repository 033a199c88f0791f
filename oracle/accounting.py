"""Oracle byte / flop accounting for the skinny product.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: Flash-LLM paper review (xllm-io), section 3 "core formulas":

* compute intensity of the dense MatMul, flops over bytes moved:
  CI = 2*M*N*K / ((M*K + K*N + M*N) * sizeof(dtype));
* for a skinny MatMul this is bounded by N (with 2-byte elements), so the
  product is memory-bound for small N;
* with sparsity beta the weight traffic shrinks while the (dense) compute does
  not;
* the Tensor-Core utilisation figures of the same section (OPT-175B MatMul,
  M = 48K, K = 12K, N = 8/16/32/64) follow from CI x bandwidth / peak.

Reading for the sparse byte count (the pages print the shrink factor (1-beta)
for the loaded data but also give every nonzero a 32-bit word): the compressed
weights cost 4 bytes per nonzero plus 4 bytes per tile offset entry, so the
algorithmic bytes of one sparse product are
    bytes = 4*nnz + 4*(T+1) + 2*K*N + 2*M*N
(B read once, C written once, padding words, split-K partials and B re-reads
earn no credit), and the useful flops are the dense-equivalent 2*M*N*K.
"""
from __future__ import annotations


def ci_dense(M: float, N: float, K: float, sizeof: int = 2) -> float:
    """Compute intensity of the dense MatMul in flop per byte."""
    return 2.0 * M * N * K / ((M * K + K * N + M * N) * sizeof)


def tc_utilisation(M: float, N: float, K: float, bandwidth: float, peak: float, sizeof: int = 2) -> float:
    """Fraction of matrix-unit peak reachable when bandwidth-bound: CI * BW / peak (capped at 1)."""
    return min(1.0, ci_dense(M, N, K, sizeof) * bandwidth / peak)


def dense_bytes(M: int, N: int, K: int, sizeof: int = 2) -> int:
    return (M * K + K * N + M * N) * sizeof


def sparse_bytes(M: int, N: int, K: int, nnz: int, tiles: int) -> int:
    """Algorithmic bytes of one sparse product with the 32-bit-word format."""
    return 4 * nnz + 4 * (tiles + 1) + 2 * K * N + 2 * M * N


def flops(M: int, N: int, K: int) -> int:
    """Dense-equivalent flops (true N, not padded)."""
    return 2 * M * N * K


def ideal_speedup_over_dense(beta: float) -> float:
    """Memory-bound speedup limit of 32-bit words over 16-bit dense weights: 1 / (2 (1 - beta))."""
    return 1.0 / (2.0 * (1.0 - beta))
