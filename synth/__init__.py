"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Nothing here computes any part of the shard-decomposed GEMM. The module turns
(seed, index) pairs into fp16 bit patterns and draws the producer's release
schedule; the recipes are stated in ``gen.c``. The shared library is built
in-tree by :func:`build` (plain ``gcc``) and loaded with ``ctypes``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

# Seeds per configuration number c = 1..5 (A, B and schedule streams).
def seeds(c: int) -> tuple[int, int, int]:
    return 0xA000 + c, 0xB000 + c, 0x5000 + c


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so next to it."""
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
        lib.synth_splitmix64.restype = ctypes.c_uint64
        lib.synth_splitmix64.argtypes = [ctypes.c_uint64]
        lib.synth_f64_to_f16.restype = ctypes.c_uint16
        lib.synth_f64_to_f16.argtypes = [ctypes.c_double]
        lib.synth_uniform.restype = ctypes.c_double
        lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fill_f16.restype = ctypes.c_int
        lib.synth_fill_f16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        lib.synth_schedule.restype = ctypes.c_int
        lib.synth_schedule.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill_f32.restype = ctypes.c_int
        lib.synth_fill_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_double, ctypes.c_double]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:
        return 4


def fill_f16(seed: int, count: int, start: int = 0) -> np.ndarray:
    """fp16 bit patterns (uint16) of elements start .. start+count-1 of stream ``seed``."""
    out = np.empty(int(count), dtype=np.uint16)
    if count:
        _load().synth_fill_f16(seed, start, out.ctypes.data, out.size, _threads())
    return out


def fill_f32(seed: int, count: int, lo: float = -1.0, hi: float = 1.0, start: int = 0) -> np.ndarray:
    """binary32 values in [lo, hi) of elements start .. start+count-1 of stream ``seed``."""
    out = np.empty(int(count), dtype=np.float32)
    if count:
        lib = _load()
        lib.synth_fill_f32(seed, start, out.ctypes.data, out.size, float(lo), float(hi))
    return out


def fd_partials(seed: int, W: int, H: int, D: int, lse_lo: float = 8.0, lse_hi: float = 16.0):
    """Per-rank Flash-Decode partials: W normalised partial outputs (H x D, uniform [-1, 1))
    and W log-sum-exp vectors (H, uniform [lse_lo, lse_hi)), both binary32. Rank s draws
    from streams seed + 2s (outputs) and seed + 2s + 1 (statistics)."""
    o = [fill_f32(seed + 2 * s, H * D).reshape(H, D) for s in range(W)]
    lse = [fill_f32(seed + 2 * s + 1, H, lse_lo, lse_hi) for s in range(W)]
    return o, lse


def matrix_f16(seed: int, rows: int, cols: int) -> np.ndarray:
    """A rows x cols row-major matrix of fp16 bits; element (r, c) uses index r*cols + c."""
    return fill_f16(seed, rows * cols).reshape(rows, cols)


def shards(a: np.ndarray, W: int) -> list[np.ndarray]:
    """Split an M x K matrix into W contiguous M x (K/W) column slices A_0 .. A_{W-1}."""
    M, K = a.shape
    if K % W:
        raise ValueError("K must be a multiple of W")
    ks = K // W
    return [np.ascontiguousarray(a[:, s * ks:(s + 1) * ks]) for s in range(W)]


def schedule(seed: int, T: int, max_delay_ns: int) -> tuple[np.ndarray, np.ndarray]:
    """Release order (int32, a permutation of 0..T-1) and cumulative release offsets (int64 ns)."""
    order = np.empty(T, dtype=np.int32)
    offs = np.empty(T, dtype=np.int64)
    rc = _load().synth_schedule(seed, T, max_delay_ns, order.ctypes.data, offs.ctypes.data)
    if rc != 0:
        raise ValueError("bad schedule arguments")
    return order, offs


def splitmix64(x: int) -> int:
    return int(_load().synth_splitmix64(x))


def f64_to_f16_bits(x: float) -> int:
    return int(_load().synth_f64_to_f16(x))


def uniform(seed: int, i: int) -> float:
    return float(_load().synth_uniform(seed, i))
