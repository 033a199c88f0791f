"""Thin Python binding of liblscd.so (the C ABI declared in include/lscd.h).

Argument marshalling only: every step of the product runs in the HIP library.  The
functions carry the C names.  Host arrays are numpy (fp16 as uint16 bit patterns);
device buffers are torch CUDA tensors, used only for their memory and the current
stream.  Importing this module loads the library and fails loudly if it is not built.

torch is imported before the library is loaded, so the library binds to the HIP runtime
torch already loaded (both carry the soname libamdhip64.so.7) and torch's stream handles
are valid in it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  (must come before loading the library, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblscd.so")

LSCD_SUCCESS = 0
LSCD_ERROR_INVALID_VALUE = 1
LSCD_ERROR_NOT_SUPPORTED = 2
LSCD_ERROR_OUT_OF_MEMORY = 3
LSCD_ERROR_INVALID_FORMAT = 4
LSCD_ERROR_HIP = 5
LSCD_DEFAULT_TILE_M = 64
LSCD_DEFAULT_TILE_K = 64
LSCD_NARROW_MAX_N = 64
LSCD_MAX_N = 65535

#: Every entry point include/lscd.h declares.
EXPORTS = ("lscd_pack_size", "lscd_pack", "lscd_default_tile_m", "lscd_encode", "lscd_encode_tiled", "lscd_encode_device",
           "lscd_pack_bitmap_size", "lscd_pack_bitmap", "lscd_encode_bitmap",
           "lscd_pack_three_level_size", "lscd_pack_three_level", "lscd_encode_three_level",
           "lscd_import", "lscd_export",
           "lscd_get_info", "lscd_spmm", "lscd_debug_decode", "lscd_attach_dense", "lscd_linear",
           "lscd_linear_path", "lscd_set_linear_crossover", "lscd_linear_model", "lscd_tune_dense", "lscd_destroy",
           "lscd_status_string", "lscd_stream_read", "lscd_spmm_noalloc", "lscd_linear_times")


class lscd_info_t(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("K", ctypes.c_int64), ("tile_m", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("num_tiles", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("nnz_padded", ctypes.c_int64), ("format_bytes", ctypes.c_int64),
                ("max_tile_words", ctypes.c_int32), ("device", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("reg_vectors", ctypes.c_int32),
                ("splits", ctypes.c_int32 * 3), ("variant", ctypes.c_int32 * 3),
                ("splits_wide", ctypes.c_int32 * 3), ("reg_vectors_wide", ctypes.c_int32),
                ("format", ctypes.c_int32)]


class LSCDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lscd_status_string(status)} ({status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python unstructured_sparse_skinny_amd/build.py` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, VP = ctypes.POINTER, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "lscd_pack_size": [VP, VP, I64, I64, I32, I32, P(I64), P(I64)],
        "lscd_pack": [VP, VP, I64, I64, I32, I32, VP, I64, VP, I64],
        "lscd_default_tile_m": [I64, I64, P(I32)],
        "lscd_encode": [VP, VP, I64, I64, P(VP)],
        "lscd_encode_tiled": [VP, VP, I64, I64, I32, I32, P(VP)],
        "lscd_encode_device": [VP, VP, I64, I64, VP, P(VP)],
        "lscd_pack_bitmap_size": [VP, VP, I64, I64, P(I64), P(I64)],
        "lscd_pack_bitmap": [VP, VP, I64, I64, VP, I64, VP, I64],
        "lscd_encode_bitmap": [VP, VP, I64, I64, P(VP)],
        "lscd_pack_three_level_size": [VP, VP, I64, I64, P(I64), P(I64)],
        "lscd_pack_three_level": [VP, VP, I64, I64, VP, I64, VP, I64],
        "lscd_encode_three_level": [VP, VP, I64, I64, P(VP)],
        "lscd_import": [VP, I64, VP, I64, I64, I32, I32, P(VP)],
        "lscd_export": [VP, VP, VP],
        "lscd_get_info": [VP, P(lscd_info_t)],
        "lscd_spmm": [VP, VP, VP, I32, VP],
        "lscd_debug_decode": [VP, VP, VP],
        "lscd_attach_dense": [VP],
        "lscd_linear": [VP, VP, VP, I32, VP],
        "lscd_linear_path": [VP, I32, P(I32)],
        "lscd_set_linear_crossover": [VP, I32],
        "lscd_linear_model": [I64, I64, I64, I64, I32, P(ctypes.c_double), P(ctypes.c_double)],
        "lscd_tune_dense": [VP, VP, VP, I32, P(ctypes.c_double), P(I32)],
        "lscd_destroy": [VP],
        "lscd_stream_read": [VP, I64, I32, VP, VP],
        "lscd_linear_times": [VP, I32, P(ctypes.c_double), P(ctypes.c_double), P(I32)],
        "lscd_spmm_noalloc": [VP, VP, VP, I32, VP],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.lscd_status_string.argtypes = [ctypes.c_int]
    lib.lscd_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lscd_status_string(status: int) -> str:
    return _lib.lscd_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != LSCD_SUCCESS:
        raise LSCDError(status, where)


class Handle:
    """Owner of an lscd_handle_t; freed by lscd_destroy (or when collected)."""

    def __init__(self, ptr: int):
        self.ptr = ptr

    def __del__(self):
        self.close()

    def close(self):
        if getattr(self, "ptr", None) and _lib is not None:   # _lib is None during interpreter teardown
            _lib.lscd_destroy(ctypes.c_void_p(self.ptr))
            self.ptr = None

    @property
    def info(self) -> dict:
        return lscd_get_info(self)


def _host_A(A16, mask):
    A16 = np.ascontiguousarray(A16, dtype=np.uint16)
    if A16.ndim != 2:
        raise ValueError("A must be a 2-D array of fp16 bit patterns")
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    if m is not None and m.shape != A16.shape:
        raise ValueError("mask must have A's shape")
    return A16, m, A16.ctypes.data, (None if m is None else m.ctypes.data)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _device_fp16(t, name, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float16 CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def lscd_pack_size(A16, mask=None, tile_m=LSCD_DEFAULT_TILE_M, tile_k=LSCD_DEFAULT_TILE_K):
    A16, m, pa, pm = _host_A(A16, mask)
    nw, nt = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.lscd_pack_size(pa, pm, A16.shape[0], A16.shape[1], tile_m, tile_k, ctypes.byref(nw),
                               ctypes.byref(nt)), "lscd_pack_size")
    return nw.value, nt.value


def lscd_pack(A16, mask=None, tile_m=LSCD_DEFAULT_TILE_M, tile_k=LSCD_DEFAULT_TILE_K):
    """Host-only encoding: returns (nonzeros uint32[nnz_padded], tile_offsets uint32[T+1])."""
    A16, m, pa, pm = _host_A(A16, mask)
    nw, nt = lscd_pack_size(A16, m, tile_m, tile_k)
    words = np.empty(max(nw, 1), dtype=np.uint32)
    offs = np.empty(nt + 1, dtype=np.uint32)
    _check(_lib.lscd_pack(pa, pm, A16.shape[0], A16.shape[1], tile_m, tile_k, words.ctypes.data, nw,
                          offs.ctypes.data, nt + 1), "lscd_pack")
    return words[:nw], offs


def lscd_default_tile_m(M: int, K: int) -> int:
    """Tile height lscd_encode / lscd_encode_device use for an M x K matrix on the current device."""
    tm = ctypes.c_int32()
    _check(_lib.lscd_default_tile_m(M, K, ctypes.byref(tm)), "lscd_default_tile_m")
    return tm.value


def lscd_encode(A16, mask=None) -> Handle:
    A16, m, pa, pm = _host_A(A16, mask)
    h = ctypes.c_void_p()
    _check(_lib.lscd_encode(pa, pm, A16.shape[0], A16.shape[1], ctypes.byref(h)), "lscd_encode")
    return Handle(h.value)


def lscd_encode_tiled(A16, mask, tile_m, tile_k) -> Handle:
    A16, m, pa, pm = _host_A(A16, mask)
    h = ctypes.c_void_p()
    _check(_lib.lscd_encode_tiled(pa, pm, A16.shape[0], A16.shape[1], tile_m, tile_k, ctypes.byref(h)),
           "lscd_encode_tiled")
    return Handle(h.value)


def lscd_pack_bitmap(A16, mask=None):
    """Host-only bitmap-tile encoding: (words uint32[nwords], tile_offsets uint32[T+1] in 16-byte units)."""
    A16, m, pa, pm = _host_A(A16, mask)
    nw, nt = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.lscd_pack_bitmap_size(pa, pm, A16.shape[0], A16.shape[1], ctypes.byref(nw), ctypes.byref(nt)),
           "lscd_pack_bitmap_size")
    words = np.empty(max(nw.value, 1), dtype=np.uint32)
    offs = np.empty(nt.value + 1, dtype=np.uint32)
    _check(_lib.lscd_pack_bitmap(pa, pm, A16.shape[0], A16.shape[1], words.ctypes.data, nw.value, offs.ctypes.data,
                                 nt.value + 1), "lscd_pack_bitmap")
    return words[:nw.value], offs


def lscd_encode_bitmap(A16, mask=None) -> Handle:
    A16, m, pa, pm = _host_A(A16, mask)
    h = ctypes.c_void_p()
    _check(_lib.lscd_encode_bitmap(pa, pm, A16.shape[0], A16.shape[1], ctypes.byref(h)), "lscd_encode_bitmap")
    return Handle(h.value)


def lscd_pack_three_level(A16, mask=None):
    """Host-only three-level encoding: (words uint32[nwords], tile_offsets uint32[T+1] in 16-byte units)."""
    A16, m, pa, pm = _host_A(A16, mask)
    nw, nt = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.lscd_pack_three_level_size(pa, pm, A16.shape[0], A16.shape[1], ctypes.byref(nw), ctypes.byref(nt)),
           "lscd_pack_three_level_size")
    words = np.empty(max(nw.value, 1), dtype=np.uint32)
    offs = np.empty(nt.value + 1, dtype=np.uint32)
    _check(_lib.lscd_pack_three_level(pa, pm, A16.shape[0], A16.shape[1], words.ctypes.data, nw.value,
                                      offs.ctypes.data, nt.value + 1), "lscd_pack_three_level")
    return words[:nw.value], offs


def lscd_encode_three_level(A16, mask=None) -> Handle:
    A16, m, pa, pm = _host_A(A16, mask)
    h = ctypes.c_void_p()
    _check(_lib.lscd_encode_three_level(pa, pm, A16.shape[0], A16.shape[1], ctypes.byref(h)),
           "lscd_encode_three_level")
    return Handle(h.value)


def lscd_encode_device(A, mask=None, stream=None) -> Handle:
    """Encode a matrix already on the GPU: A float16 [M][K], mask uint8/bool [M][K] or None."""
    if not isinstance(A, torch.Tensor) or not A.is_cuda or A.dim() != 2 or not A.is_contiguous() or \
            A.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise ValueError("A must be a contiguous 2-D CUDA tensor of fp16 (or 16-bit patterns)")
    pm = None
    if mask is not None:
        if not isinstance(mask, torch.Tensor) or not mask.is_cuda or tuple(mask.shape) != tuple(A.shape) or \
                not mask.is_contiguous() or mask.dtype not in (torch.uint8, torch.bool):
            raise ValueError("mask must be a contiguous uint8/bool CUDA tensor of A's shape")
        pm = ctypes.c_void_p(mask.data_ptr())
    h = ctypes.c_void_p()
    _check(_lib.lscd_encode_device(ctypes.c_void_p(A.data_ptr()), pm, A.shape[0], A.shape[1], _stream(stream),
                                   ctypes.byref(h)), "lscd_encode_device")
    return Handle(h.value)


def lscd_import(nonzeros, tile_offsets, M, K, tile_m=LSCD_DEFAULT_TILE_M, tile_k=LSCD_DEFAULT_TILE_K) -> Handle:
    w = np.ascontiguousarray(nonzeros, dtype=np.uint32)
    o = np.ascontiguousarray(tile_offsets, dtype=np.uint32)
    h = ctypes.c_void_p()
    _check(_lib.lscd_import(w.ctypes.data if w.size else None, w.size, o.ctypes.data, M, K, tile_m, tile_k,
                            ctypes.byref(h)), "lscd_import")
    return Handle(h.value)


def lscd_get_info(h: Handle) -> dict:
    info = lscd_info_t()
    _check(_lib.lscd_get_info(ctypes.c_void_p(h.ptr), ctypes.byref(info)), "lscd_get_info")
    out = {name: getattr(info, name) for name, _ in lscd_info_t._fields_}
    out["splits"], out["variant"] = list(info.splits), list(info.variant)
    out["splits_wide"] = list(info.splits_wide)
    return out


def npad_index(N: int) -> int:
    """Index into lscd_info_t.splits / .variant for a batch width N."""
    return 0 if N <= 16 else (1 if N <= 32 else 2)


def lscd_export(h: Handle):
    info = lscd_get_info(h)
    words = np.empty(max(info["nnz_padded"], 1), dtype=np.uint32)
    offs = np.empty(info["num_tiles"] + 1, dtype=np.uint32)
    _check(_lib.lscd_export(ctypes.c_void_p(h.ptr), words.ctypes.data, offs.ctypes.data), "lscd_export")
    return words[:info["nnz_padded"]], offs


def lscd_spmm(h: Handle, B, C, stream=None):
    """C[N][M] = A . B^T for B[N][K] (float16 CUDA tensors), enqueued on `stream`."""
    info = lscd_get_info(h)
    N = int(B.shape[0]) if isinstance(B, torch.Tensor) and B.dim() == 2 else -1
    pb = _device_fp16(B, "B", (N, info["K"]))
    pc = _device_fp16(C, "C", (N, info["M"]))
    _check(_lib.lscd_spmm(ctypes.c_void_p(h.ptr), pb, pc, N, _stream(stream)), "lscd_spmm")
    return C


def lscd_spmm_noalloc(h: Handle, B, C, stream=None):
    """lscd_spmm with its split-K partial sums in the library's static per-GPU array instead of
    the handle's workspace (for callers that cannot allocate; calls on one GPU must not overlap)."""
    info = lscd_get_info(h)
    N = int(B.shape[0]) if isinstance(B, torch.Tensor) and B.dim() == 2 else -1
    pb = _device_fp16(B, "B", (N, info["K"]))
    pc = _device_fp16(C, "C", (N, info["M"]))
    _check(_lib.lscd_spmm_noalloc(ctypes.c_void_p(h.ptr), pb, pc, N, _stream(stream)), "lscd_spmm_noalloc")
    return C


def lscd_attach_dense(h: Handle):
    _check(_lib.lscd_attach_dense(ctypes.c_void_p(h.ptr)), "lscd_attach_dense")


def lscd_linear(h: Handle, B, C, stream=None):
    """lscd_spmm, or the dense GEMM on the attached dense copy when lscd_linear_path says so."""
    info = lscd_get_info(h)
    N = int(B.shape[0]) if isinstance(B, torch.Tensor) and B.dim() == 2 else -1
    pb = _device_fp16(B, "B", (N, info["K"]))
    pc = _device_fp16(C, "C", (N, info["M"]))
    _check(_lib.lscd_linear(ctypes.c_void_p(h.ptr), pb, pc, N, _stream(stream)), "lscd_linear")
    return C


def lscd_tune_dense(h: Handle, B, C):
    """Time hipBLASLt's heuristic candidates for the dense GEMM at width N = B.shape[0] and keep
    the fastest for lscd_linear; returns (best microseconds per GEMM, candidates timed)."""
    info = lscd_get_info(h)
    N = int(B.shape[0]) if isinstance(B, torch.Tensor) and B.dim() == 2 else -1
    pb = _device_fp16(B, "B", (N, info["K"]))
    pc = _device_fp16(C, "C", (N, info["M"]))
    us, n = ctypes.c_double(), ctypes.c_int32()
    _check(_lib.lscd_tune_dense(ctypes.c_void_p(h.ptr), pb, pc, N, ctypes.byref(us), ctypes.byref(n)),
           "lscd_tune_dense")
    return us.value, n.value


def lscd_linear_times(h: Handle, N: int):
    """The (sparse, dense) microseconds lscd_linear compares for N, and whether both were
    measured by lscd_tune_dense (else model predictions)."""
    ts, td, m = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _check(_lib.lscd_linear_times(ctypes.c_void_p(h.ptr), N, ctypes.byref(ts), ctypes.byref(td), ctypes.byref(m)),
           "lscd_linear_times")
    return ts.value, td.value, bool(m.value)


def lscd_linear_path(h: Handle, N: int) -> int:
    p = ctypes.c_int32()
    _check(_lib.lscd_linear_path(ctypes.c_void_p(h.ptr), N, ctypes.byref(p)), "lscd_linear_path")
    return p.value


def lscd_set_linear_crossover(h: Handle, n_max_sparse: int):
    _check(_lib.lscd_set_linear_crossover(ctypes.c_void_p(h.ptr), n_max_sparse), "lscd_set_linear_crossover")


def lscd_linear_model(M: int, K: int, nnz_padded: int, num_tiles: int, N: int):
    """(t_sparse_us, t_dense_us) predicted by the selection cost model (host only)."""
    ts, td = ctypes.c_double(), ctypes.c_double()
    _check(_lib.lscd_linear_model(M, K, nnz_padded, num_tiles, N, ctypes.byref(ts), ctypes.byref(td)),
           "lscd_linear_model")
    return ts.value, td.value


def lscd_debug_decode(h: Handle, A_dense, stream=None):
    info = lscd_get_info(h)
    pa = _device_fp16(A_dense, "A_dense", (info["M"], info["K"]))
    _check(_lib.lscd_debug_decode(ctypes.c_void_p(h.ptr), pa, _stream(stream)), "lscd_debug_decode")
    return A_dense


def lscd_stream_read(src, nbytes: int, blocks_per_cu: int, sink, stream=None):
    """Measurement reference: stream `nbytes` of the device tensor `src` with the product's loads
    (see include/lscd.h); `sink` is a device tensor of at least 4 bytes."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and isinstance(sink, torch.Tensor) and sink.is_cuda):
        raise ValueError("src and sink must be CUDA tensors")
    if nbytes > src.numel() * src.element_size() or sink.numel() * sink.element_size() < 4:
        raise ValueError("buffer too small")
    _check(_lib.lscd_stream_read(ctypes.c_void_p(src.data_ptr()), int(nbytes), int(blocks_per_cu),
                                 ctypes.c_void_p(sink.data_ptr()), _stream(stream)), "lscd_stream_read")


def lscd_destroy(h: Handle):
    h.close()
