"""Pins for the oracle's byte/flop accounting (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import accounting as acc


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "ci_utilisation.json")) as f:
        return json.load(f)


def test_hand_worked_ci(golden_dir):
    g = _golden(golden_dir)
    for h in g["hand_ci"]:
        assert abs(acc.ci_dense(h["M"], h["N"], h["K"]) - float(Fraction(h["ci"]))) < 1e-12


def test_ci_bounded_by_n_and_tends_to_n():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        M, K = rng.integers(1, 1 << 17, size=2)
        N = int(rng.integers(1, 512))
        assert acc.ci_dense(M, N, K) < N
    assert acc.ci_dense(1 << 30, 16, 1 << 30) > 16 * (1 - 1e-6)


def test_page_utilisation_is_bracketed(golden_dir):
    """CI x bandwidth / peak brackets the utilisation printed for the OPT-175B MatMul."""
    g = _golden(golden_dir)
    lo_bw, hi_bw = g["a100_bandwidth_range"]
    for n, pct in g["page_utilisation_percent"].items():
        lo = 100 * acc.tc_utilisation(g["M"], int(n), g["K"], lo_bw, g["a100_peak_flops"])
        hi = 100 * acc.tc_utilisation(g["M"], int(n), g["K"], hi_bw, g["a100_peak_flops"])
        assert lo - 0.05 <= pct <= hi + 0.05, (n, lo, pct, hi)


def test_hand_worked_sparse_bytes(golden_dir):
    for h in _golden(golden_dir)["hand_sparse_bytes"]:
        assert acc.sparse_bytes(h["M"], h["N"], h["K"], h["nnz"], h["tiles"]) == h["bytes"]


def test_dense_limit_and_page_speedups(golden_dir):
    # at 50% sparsity 32-bit words move exactly the dense weight bytes
    M, K, N = 4096, 4096, 16
    nnz = M * K // 2
    assert acc.sparse_bytes(M, N, K, nnz, 0) - 4 == acc.dense_bytes(M, N, K)
    assert acc.ideal_speedup_over_dense(0.5) == 1.0
    # the measured speedups over the dense library stay under the memory-bound ideal
    for beta, s in _golden(golden_dir)["page_speedup_vs_dense"].items():
        assert s <= acc.ideal_speedup_over_dense(float(beta))
    assert acc.flops(3, 2, 5) == 60
