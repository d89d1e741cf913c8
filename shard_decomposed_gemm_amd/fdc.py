"""ctypes binding of the Flash-Decode combine C-ABI (include/fdcombine.h).

Argument marshalling only: every step runs in libagemm.so's kernels, and the
binding raises when the library is missing.
"""
from __future__ import annotations

import ctypes

from . import agemm
from .agemm import F16, F32, OK, AgemmError, _ptr, _stream_handle, make_schedule, status_string

EXPORTED = (
    "fdc_create", "fdc_destroy", "fdc_tiles", "fdc_produce", "fdc_run_fused", "fdc_run_bsp",
    "fdc_set_spin_timeout_us", "fdc_timing_begin", "fdc_timing_end", "fdc_check", "fdc_last_error",
    "fdc_streams",
)

_ready = False


def load() -> ctypes.CDLL:
    """libagemm.so with the fdc_* signatures set."""
    global _ready
    lib = agemm.load()
    if not _ready:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.fdc_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int]
        lib.fdc_destroy.argtypes = [vp]
        lib.fdc_tiles.argtypes = [vp, ctypes.POINTER(i32)]
        lib.fdc_produce.argtypes = [vp, vp, vp, ctypes.POINTER(agemm.Schedule), vp]
        lib.fdc_run_fused.argtypes = [vp, vp, vp]
        lib.fdc_run_bsp.argtypes = [vp, vp, vp, vp, ctypes.POINTER(agemm.Schedule), ctypes.c_int, vp]
        lib.fdc_set_spin_timeout_us.argtypes = [vp, i64]
        lib.fdc_timing_begin.argtypes = [vp, i32]
        lib.fdc_timing_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
        lib.fdc_check.argtypes = [vp]
        lib.fdc_streams.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        lib.fdc_last_error.argtypes = [vp]
        lib.fdc_last_error.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "fdc_last_error":
                getattr(lib, name).restype = ctypes.c_int
        _ready = True
    return lib


class FdCombine:
    """One shape of the flag-gated Flash-Decode combine (owns the inboxes and flags).

    Partials per rank s: o_parts[s] (H x D float32, normalised partial output)
    and lse_parts[s] (H float32, log-sum-exp of the rank's scores)."""

    def __init__(self, W: int, H: int, D: int, heads_per_tile: int = 16, out_dtype: str = "f16"):
        lib = load()
        self._lib = lib
        self.W, self.H, self.D, self.HT = int(W), int(H), int(D), int(heads_per_tile)
        self.out_dtype = out_dtype
        code = {"f16": F16, "f32": F32}.get(out_dtype)
        if code is None:
            raise ValueError("out_dtype must be 'f16' or 'f32'")
        h = ctypes.c_void_p()
        rc = lib.fdc_create(ctypes.byref(h), self.W, self.H, self.D, self.HT, code)
        if rc != OK:
            raise AgemmError(rc, f"fdc_create: {status_string(rc)}")
        self._h = h
        t = ctypes.c_int32()
        lib.fdc_tiles(h, ctypes.byref(t))
        self.t = t.value

    def _raise(self, rc: int, what: str):
        if rc != OK:
            msg = self._lib.fdc_last_error(self._h).decode()
            raise AgemmError(rc, f"{what}: {msg or status_string(rc)}")

    def _parts(self, o_parts, lse_parts):
        import torch
        if len(o_parts) != self.W or len(lse_parts) != self.W:
            raise ValueError(f"expected {self.W} partials")
        o = [_ptr(x, f"o_parts[{i}]", torch.float32, (self.H, self.D)) for i, x in enumerate(o_parts)]
        lse = [_ptr(x, f"lse_parts[{i}]", torch.float32, (self.H,)) for i, x in enumerate(lse_parts)]
        return (ctypes.c_void_p * self.W)(*o), (ctypes.c_void_p * self.W)(*lse)

    def _out(self, O):
        import torch
        dt = torch.float16 if self.out_dtype == "f16" else torch.float32
        return _ptr(O, "O", dt, (self.H, self.D))

    @staticmethod
    def _sched(schedule):
        if schedule is None:
            return None, None
        keep = make_schedule(*schedule)
        return ctypes.byref(keep[0]), keep

    def produce(self, o_parts, lse_parts, schedule=None, stream=None):
        o, lse = self._parts(o_parts, lse_parts)
        sp, keep = self._sched(schedule)
        self._raise(self._lib.fdc_produce(self._h, o, lse, sp, _stream_handle(stream)), "fdc_produce")
        del keep

    def run_fused(self, O, stream=None):
        self._raise(self._lib.fdc_run_fused(self._h, self._out(O), _stream_handle(stream)), "fdc_run_fused")

    def run_bsp(self, o_parts, lse_parts, O, schedule=None, host_sync: bool = True, stream=None):
        o, lse = self._parts(o_parts, lse_parts)
        sp, keep = self._sched(schedule)
        self._raise(self._lib.fdc_run_bsp(self._h, o, lse, self._out(O), sp, 1 if host_sync else 0,
                                          _stream_handle(stream)), "fdc_run_bsp")
        del keep

    def streams(self):
        """fdc_streams: (producer, consumer) torch streams verified to run concurrently,
        owned by the context (valid until close())."""
        import torch
        if getattr(self, "_pair", None) is None:
            p, c = ctypes.c_void_p(), ctypes.c_void_p()
            self._raise(self._lib.fdc_streams(self._h, ctypes.byref(p), ctypes.byref(c)), "fdc_streams")
            self._pair = (torch.cuda.ExternalStream(p.value), torch.cuda.ExternalStream(c.value))
        return self._pair

    def set_spin_timeout_us(self, us: int):
        self._raise(self._lib.fdc_set_spin_timeout_us(self._h, int(us)), "fdc_set_spin_timeout_us")

    def timing_begin(self, max_launches: int):
        self._raise(self._lib.fdc_timing_begin(self._h, int(max_launches)), "fdc_timing_begin")

    def timing_end(self):
        cap = 100000
        buf = (ctypes.c_float * cap)()
        n = ctypes.c_int32()
        self._raise(self._lib.fdc_timing_end(self._h, buf, cap, ctypes.byref(n)), "fdc_timing_end")
        return [float(buf[i]) for i in range(min(n.value, cap))]

    def check(self):
        self._raise(self._lib.fdc_check(self._h), "fdc_check")

    def close(self):
        if getattr(self, "_h", None):
            if getattr(self, "_pair", None) is not None:
                import torch
                torch.cuda.synchronize()
                self._pair = None
            self._lib.fdc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
