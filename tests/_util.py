"""Shared helpers for the tests (not collected)."""
import contextlib
import os
import sys

import numpy as np

# Parity bar for floating-point results of the product (applied to the compared set):
#   max |C_gpu - C_oracle| <= 1e-2 * max |C_oracle|   and   ||C_gpu - C_oracle||_F <= 2e-3 * ||C_oracle||_F
MAX_REL = 1e-2
FRO_REL = 2e-3


def gate_errors(C16_bits: np.ndarray, C64: np.ndarray):
    """(max-abs error relative to max |C64|, relative Frobenius error) of fp16 bits vs fp64."""
    c = np.asarray(C16_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    d = c - C64
    scale = np.abs(C64).max()
    fro = np.linalg.norm(C64)
    max_rel = float(np.abs(d).max() / scale) if scale > 0 else float(np.abs(d).max())
    fro_rel = float(np.linalg.norm(d) / fro) if fro > 0 else float(np.linalg.norm(d))
    return max_rel, fro_rel


def assert_gates(C16_bits, C64, what=""):
    mr, fr = gate_errors(C16_bits, C64)
    assert np.isfinite(mr) and np.isfinite(fr), what
    assert mr <= MAX_REL and fr <= FRO_REL, f"{what}: max_rel={mr:.3e} fro_rel={fr:.3e}"
    return mr, fr


@contextlib.contextmanager
def env(**kw):
    old = {k: os.environ.get(k) for k in kw}
    try:
        for k, v in kw.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(v)
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def say(*a):
    """Print and flush (names the case before a GPU step)."""
    print(*a, flush=True)
    sys.stdout.flush()
