"""Plain C oracle (`spmm_loop.c`): Tiled-CSL decode and the fp64 triple loop.

TEST INFRASTRUCTURE ONLY (see the package header).

The C source states its sources and readings; this module builds it with gcc (OpenMP, no
fast-math, no FMA contraction, so every sum runs over k in ascending order exactly as
written) into `liboracle_loop.so` beside it, and calls it through ctypes.  The same
definitions as `tiled_csl.decode` and `spmm.spmm_f64`, written a second time as plain loops:
the tests pin the two against each other and against the hand-worked goldens, and
bench.py times this one as the CPU baseline.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spmm_loop.c")
LIB = os.path.join(HERE, "liboracle_loop.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall"]

_lib = None


def build() -> str:
    """Compile spmm_loop.c into liboracle_loop.so (every call)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_decode_tiled_csl.argtypes = [p, i64, p, i64, i64, ctypes.c_int32, ctypes.c_int32, p, p]
        lib.oracle_decode_tiled_csl.restype = ctypes.c_int
        lib.oracle_spmm_loop.argtypes = [p, p, i64, i64, i64, p, i64, p, ctypes.c_int]
        lib.oracle_spmm_loop.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def decode(words: np.ndarray, offsets: np.ndarray, M: int, K: int, tile_m: int, tile_k: int) -> np.ndarray:
    """Dense A[M][K] (fp16 bits) of a Tiled-CSL encoding; raises ValueError(code) if invalid."""
    lib = _load()
    w = np.ascontiguousarray(words, dtype=np.uint32)
    o = np.ascontiguousarray(offsets, dtype=np.uint32)
    MB, KT = -(-M // tile_m), -(-K // tile_k)
    if o.size != MB * KT + 1:
        raise ValueError("offsets must have tiles + 1 entries")
    dense = np.empty((M, K), dtype=np.uint16)
    seen = np.empty((M, K), dtype=np.uint8)
    code = lib.oracle_decode_tiled_csl(_ptr(w), w.size, _ptr(o), M, K, tile_m, tile_k, _ptr(dense), _ptr(seen))
    if code != 0:
        raise ValueError(f"invalid Tiled-CSL encoding (rule {code})")
    return dense


def spmm(A_dense: np.ndarray, B16: np.ndarray, rows=None, threads: int = 0) -> np.ndarray:
    """out[n][r] = sum_k A[rows[r]][k] * B[n][k] in fp64 (k ascending) for dense fp16-bit A."""
    lib = _load()
    A = np.ascontiguousarray(A_dense, dtype=np.uint16)
    B = np.ascontiguousarray(B16, dtype=np.uint16)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    r = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= M):
        raise ValueError("row index outside A")
    out = np.empty((N, r.size), dtype=np.float64)
    if lib.oracle_spmm_loop(_ptr(A), _ptr(B), M, K, N, _ptr(r), r.size, _ptr(out), int(threads)) != 0:
        raise MemoryError("oracle_spmm_loop: out of memory")
    return out


def max_threads() -> int:
    """Threads an OpenMP region of the C oracle uses by default."""
    return int(_load().oracle_max_threads())
