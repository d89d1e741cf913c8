"""CPU oracle for the shard-decomposed GEMM (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path never does. The
arithmetic lives in ``oracle.c`` (plain C, binary64); this file only builds
and marshals. Every function here follows the AG+GEMM core identity of the
"Eliminating Multi-GPU Performance Taxes" analysis page: C = sum over shards s
of A_s . B[sK/W:(s+1)K/W, :], shards visited in ascending order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lpthread"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_sharded_gemm.restype = ctypes.c_int
        lib.oracle_sharded_gemm.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, ctypes.c_int]
        lib.oracle_shard_partial.restype = ctypes.c_int
        lib.oracle_shard_partial.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp, vp, ctypes.c_int]
        lib.oracle_sharded_gemm_entries.restype = ctypes.c_int
        lib.oracle_sharded_gemm_entries.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, i64, vp, vp, vp]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:
        return 4


def _check_inputs(a_shards, b):
    W = len(a_shards)
    if W < 1:
        raise ValueError("need at least one shard")
    M, KS = a_shards[0].shape
    for a in a_shards:
        if a.dtype != np.uint16 or a.shape != (M, KS) or not a.flags.c_contiguous:
            raise ValueError("shards must be C-contiguous uint16 (fp16 bits) arrays of one shape")
    if b.dtype != np.uint16 or b.ndim != 2 or b.shape[0] != W * KS or not b.flags.c_contiguous:
        raise ValueError("B must be a C-contiguous uint16 (fp16 bits) array of shape (W*KS, N)")
    return W, M, W * KS, b.shape[1]


def _ptrs(a_shards):
    arr = (ctypes.c_void_p * len(a_shards))(*[a.ctypes.data for a in a_shards])
    return arr


def f16_to_f64(bits: int) -> float:
    return float(_load().oracle_f16_to_f64(int(bits) & 0xFFFF))


def sharded_gemm(a_shards, b, nthreads: int | None = None) -> np.ndarray:
    """C = sum_s A_s . B_s in binary64 (M x N)."""
    W, M, K, N = _check_inputs(a_shards, b)
    c = np.empty((M, N), dtype=np.float64)
    ptrs = _ptrs(a_shards)
    rc = _load().oracle_sharded_gemm(W, M, K, N, ptrs, b.ctypes.data, c.ctypes.data, nthreads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_sharded_gemm failed ({rc})")
    return c


def shard_partial(a_shards, b, s: int, nthreads: int | None = None) -> np.ndarray:
    """P_s = A_s . B[s*KS:(s+1)*KS, :] in binary64 (M x N)."""
    W, M, K, N = _check_inputs(a_shards, b)
    p = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_shard_partial(W, s, M, K, N, _ptrs(a_shards), b.ctypes.data, p.ctypes.data,
                                      nthreads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_shard_partial failed ({rc})")
    return p


def sharded_gemm_entries(a_shards, b, rows, cols) -> np.ndarray:
    """C[rows[i], cols[i]] by the same definition, one entry at a time."""
    W, M, K, N = _check_inputs(a_shards, b)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D of equal length")
    out = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_sharded_gemm_entries(W, M, K, N, _ptrs(a_shards), b.ctypes.data, rows.size,
                                             rows.ctypes.data, cols.ctypes.data, out.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_sharded_gemm_entries failed ({rc})")
    return out


def tolerance(K: int) -> float:
    """Parity bound for inputs uniform in [-1, 1]: max |C_gpu - C_oracle| <= 1e-3 * sqrt(K)."""
    return 1e-3 * float(np.sqrt(K))
