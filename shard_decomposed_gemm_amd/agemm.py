"""ctypes binding of libagemm.so (include/agemm.h), argument marshalling only.

Torch tensors are used for device memory and streams: this module passes
their data pointers and HIP stream handles to the C-ABI and never computes
anything itself. If the library has not been built the import of this
module still works, but any use raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libagemm.so")

OK, EINVAL, ESHAPE, ENOMEM, EHIP, ETIMEOUT, ESTATE = range(7)
F16, F32 = 0, 1

EXPORTED = (
    "agemm_create", "agemm_destroy", "agemm_tiles", "agemm_consumer_kernel", "agemm_consumer_grid", "agemm_mfma_plan", "agemm_produce", "agemm_run_fused",
    "agemm_run_bsp", "agemm_run_pull", "agemm_set_order", "agemm_set_spin_timeout_us", "agemm_timing_begin", "agemm_timing_end",
    "agemm_consumer_info", "agemm_set_strict_acquire", "agemm_pull_noalloc", "agemm_streams",
    "agemm_check", "agemm_device_info", "agemm_probe_mfma", "agemm_probe_read",
    "agemm_last_error", "agemm_status_string",
)


class AgemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Schedule(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("order", ctypes.c_void_p), ("offset_ns", ctypes.c_void_p)]


class ConsumerDesc(ctypes.Structure):
    """agemm_consumer_desc: the consumer launch a context's calls make."""
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "tile_config", "block_m", "block_n", "tiles", "grid", "split",
                                               "b_nontemporal", "tiles_per_wg", "ranges", "a_panels")]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libagemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.agemm_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, i64, i64, i64, ctypes.c_int, i64]
    lib.agemm_destroy.argtypes = [vp]
    lib.agemm_tiles.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.agemm_consumer_kernel.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.agemm_consumer_grid.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.agemm_mfma_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.agemm_produce.argtypes = [vp, vp, ctypes.POINTER(Schedule), vp]
    lib.agemm_run_fused.argtypes = [vp, vp, vp, vp]
    lib.agemm_run_bsp.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Schedule), ctypes.c_int, vp]
    lib.agemm_run_pull.argtypes = [vp, vp, vp, vp, vp]
    lib.agemm_set_order.argtypes = [vp, ctypes.c_int]
    lib.agemm_consumer_info.argtypes = [vp, ctypes.POINTER(ConsumerDesc)]
    lib.agemm_set_strict_acquire.argtypes = [vp, ctypes.c_int]
    lib.agemm_streams.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.agemm_pull_noalloc.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp]
    lib.agemm_set_spin_timeout_us.argtypes = [vp, i64]
    lib.agemm_timing_begin.argtypes = [vp, i32]
    lib.agemm_timing_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
    lib.agemm_check.argtypes = [vp]
    lib.agemm_device_info.argtypes = [ctypes.POINTER(i32)] * 4
    lib.agemm_probe_mfma.argtypes = [i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    lib.agemm_probe_read.argtypes = [vp, i64, i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    lib.agemm_last_error.argtypes = [vp]
    lib.agemm_last_error.restype = ctypes.c_char_p
    lib.agemm_status_string.argtypes = [ctypes.c_int]
    lib.agemm_status_string.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("agemm_last_error", "agemm_status_string"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def mfma_plan(M: int, N: int, K: int, W: int, num_cus: int, tile_config: int = -1, split_mode: int = -1):
    """Host-only plan of the MFMA consumer (agemm_mfma_plan): (tile config, grid, split)."""
    cfg, grid, split = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = load().agemm_mfma_plan(int(M), int(N), int(K), int(W), int(num_cus), int(tile_config), int(split_mode),
                                ctypes.byref(cfg), ctypes.byref(grid), ctypes.byref(split))
    if rc != OK:
        raise AgemmError(rc, f"agemm_mfma_plan: {status_string(rc)}")
    return cfg.value, grid.value, bool(split.value)


def pull_noalloc(a_shards, B, C, stream=None) -> int:
    """agemm_pull_noalloc: Pull GEMM with no context and no device allocation. Returns
    the status code (the caller decides; there is no context to hold an error text)."""
    import torch
    W = len(a_shards)
    M, KS = a_shards[0].shape
    K, N = B.shape
    code = {torch.float16: F16, torch.float32: F32}.get(C.dtype)
    if code is None:
        raise TypeError("C must be float16 or float32")
    arr = (ctypes.c_void_p * W)(*[_ptr(a, f"a_shards[{i}]", torch.float16, (M, KS)) for i, a in enumerate(a_shards)])
    return load().agemm_pull_noalloc(W, M, K, N, code, arr, _ptr(B, "B", torch.float16, (K, N)),
                                     _ptr(C, "C", None, (M, N)), _stream_handle(stream))


def status_string(code: int) -> str:
    return load().agemm_status_string(code).decode()


def device_info() -> dict:
    """agemm_device_info: compute units, clocks (kHz) and memory bus width (bits)."""
    v = [ctypes.c_int32() for _ in range(4)]
    rc = load().agemm_device_info(*[ctypes.byref(x) for x in v])
    if rc != OK:
        raise AgemmError(rc, f"agemm_device_info: {status_string(rc)}")
    return dict(zip(("cus", "clock_khz", "mem_clock_khz", "bus_bits"), (x.value for x in v)))


def probe_mfma(warmup: int = 100, launches: int = 30, stream=None) -> float:
    """agemm_probe_mfma: register-only fp16 MFMA throughput of the device, TFLOP/s."""
    import torch
    out = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    v = ctypes.c_double()
    rc = load().agemm_probe_mfma(int(warmup), int(launches), out.data_ptr(), _stream_handle(stream), ctypes.byref(v))
    if rc != OK:
        raise AgemmError(rc, f"agemm_probe_mfma: {status_string(rc)}")
    return v.value


def probe_read(buf, warmup: int = 10, launches: int = 20, stream=None) -> float:
    """agemm_probe_read over the bytes of a contiguous device tensor: streaming read, GB/s."""
    import torch
    out = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    nbytes = buf.numel() * buf.element_size()
    v = ctypes.c_double()
    rc = load().agemm_probe_read(_ptr(buf, "buf"), ctypes.c_int64(nbytes), int(warmup), int(launches),
                                 out.data_ptr(), _stream_handle(stream), ctypes.byref(v))
    if rc != OK:
        raise AgemmError(rc, f"agemm_probe_read: {status_string(rc)}")
    return v.value


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def _ptr(t, what: str, dtype=None, shape=None) -> int:
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def make_schedule(order, offset_ns):
    """Host-side agemm_schedule (the arrays are kept alive by the returned tuple)."""
    order = np.ascontiguousarray(order, dtype=np.int32)
    offs = np.ascontiguousarray(offset_ns, dtype=np.int64)
    s = Schedule(order.size, order.ctypes.data, offs.ctypes.data)
    return (s, order, offs)


class Context:
    """One shape of the flag-gated shard-decomposed GEMM (owns inbox and flags)."""

    def __init__(self, W: int, M: int, K: int, N: int, c_dtype: str = "f16", flag_ktile: int = 0):
        lib = load()
        self._lib = lib
        self.W, self.M, self.K, self.N = int(W), int(M), int(K), int(N)
        self.KS = self.K // self.W if self.W else 0
        self.c_dtype = c_dtype
        code = {"f16": F16, "f32": F32}.get(c_dtype)
        if code is None:
            raise ValueError("c_dtype must be 'f16' or 'f32'")
        h = ctypes.c_void_p()
        rc = lib.agemm_create(ctypes.byref(h), self.W, self.M, self.K, self.N, code, int(flag_ktile))
        if rc != OK:
            raise AgemmError(rc, f"agemm_create: {status_string(rc)}")
        self._h = h
        bkf, kt, t = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        lib.agemm_tiles(h, ctypes.byref(bkf), ctypes.byref(kt), ctypes.byref(t))
        self.bkf, self.kt, self.t = bkf.value, kt.value, t.value
        kind, cfg = ctypes.c_int32(), ctypes.c_int32()
        lib.agemm_consumer_kernel(h, ctypes.byref(kind), ctypes.byref(cfg))
        # consumer kernel of this context: ("mfma", tile config) or ("small_m", -1)
        self.consumer = ("small_m" if kind.value == 1 else "mfma", cfg.value)
        grid, split = ctypes.c_int32(), ctypes.c_int32()
        lib.agemm_consumer_grid(h, ctypes.byref(grid), ctypes.byref(split))
        # MFMA consumer's workgroups (-1 for small-M) and whether it runs the stream-K split
        self.grid, self.split = grid.value, bool(split.value)

    # -- helpers
    def _raise(self, rc: int, what: str):
        if rc != OK:
            msg = self._lib.agemm_last_error(self._h).decode()
            raise AgemmError(rc, f"{what}: {msg or status_string(rc)}")

    def _shards(self, a_shards):
        import torch
        if len(a_shards) != self.W:
            raise ValueError(f"expected {self.W} shards, got {len(a_shards)}")
        ptrs = [_ptr(a, f"a_shards[{i}]", torch.float16, (self.M, self.KS)) for i, a in enumerate(a_shards)]
        return (ctypes.c_void_p * self.W)(*ptrs)

    def _bc(self, B, C):
        import torch
        cdt = torch.float16 if self.c_dtype == "f16" else torch.float32
        return (_ptr(B, "B", torch.float16, (self.K, self.N)), _ptr(C, "C", cdt, (self.M, self.N)))

    @staticmethod
    def _sched(schedule):
        if schedule is None:
            return None, None
        keep = make_schedule(*schedule) if not isinstance(schedule[0], Schedule) else schedule
        return ctypes.byref(keep[0]), keep

    # -- the C-ABI
    def produce(self, a_shards, schedule=None, stream=None):
        arr = self._shards(a_shards)
        sp, keep = self._sched(schedule)
        self._raise(self._lib.agemm_produce(self._h, arr, sp, _stream_handle(stream)), "agemm_produce")
        del keep

    def run_fused(self, B, C, stream=None):
        b, c = self._bc(B, C)
        self._raise(self._lib.agemm_run_fused(self._h, b, c, _stream_handle(stream)), "agemm_run_fused")

    def run_bsp(self, a_shards, B, C, schedule=None, host_sync: bool = True, stream=None):
        arr = self._shards(a_shards)
        b, c = self._bc(B, C)
        sp, keep = self._sched(schedule)
        self._raise(self._lib.agemm_run_bsp(self._h, arr, b, c, sp, 1 if host_sync else 0, _stream_handle(stream)),
                    "agemm_run_bsp")
        del keep

    def run_pull(self, a_shards, B, C, stream=None):
        arr = self._shards(a_shards)
        b, c = self._bc(B, C)
        self._raise(self._lib.agemm_run_pull(self._h, arr, b, c, _stream_handle(stream)), "agemm_run_pull")

    def set_order(self, order: str):
        """Flag-tile order of later run_fused calls: "shard" or "arrival" (agemm_set_order)."""
        code = {"shard": 0, "arrival": 1}.get(order)
        if code is None:
            raise ValueError("order must be 'shard' or 'arrival'")
        self._raise(self._lib.agemm_set_order(self._h, code), "agemm_set_order")

    def consumer_info(self) -> dict:
        """agemm_consumer_info: the consumer launch of this context's calls (under its current order)."""
        d = ConsumerDesc()
        self._raise(self._lib.agemm_consumer_info(self._h, ctypes.byref(d)), "agemm_consumer_info")
        out = {name: getattr(d, name) for name, _ in ConsumerDesc._fields_}
        out["kind"] = "small_m" if d.kind == 1 else "mfma"
        return out

    def streams(self):
        """agemm_streams: (producer, consumer) torch streams verified to run concurrently,
        owned by the context (valid until close())."""
        import torch
        if getattr(self, "_pair", None) is None:
            p, c = ctypes.c_void_p(), ctypes.c_void_p()
            self._raise(self._lib.agemm_streams(self._h, ctypes.byref(p), ctypes.byref(c)), "agemm_streams")
            self._pair = (torch.cuda.ExternalStream(p.value), torch.cuda.ExternalStream(c.value))
        return self._pair

    def set_strict_acquire(self, strict: bool):
        """Flag-wait mode of later run_fused calls: False = no fence, True = agent-scope acquire."""
        self._raise(self._lib.agemm_set_strict_acquire(self._h, 1 if strict else 0), "agemm_set_strict_acquire")

    def set_spin_timeout_us(self, us: int):
        self._raise(self._lib.agemm_set_spin_timeout_us(self._h, int(us)), "agemm_set_spin_timeout_us")

    def timing_begin(self, max_launches: int):
        """Time the next consumer kernel launches (events attached to their dispatch)."""
        self._raise(self._lib.agemm_timing_begin(self._h, int(max_launches)), "agemm_timing_begin")

    def timing_end(self):
        """Synchronise on the timed launches; their kernel durations in microseconds."""
        cap = 100000
        buf = (ctypes.c_float * cap)()
        n = ctypes.c_int32()
        self._raise(self._lib.agemm_timing_end(self._h, buf, cap, ctypes.byref(n)), "agemm_timing_end")
        return [float(buf[i]) for i in range(min(n.value, cap))]

    def check(self):
        """Raises AgemmError(ETIMEOUT) if a consumer timed out (call after synchronising)."""
        self._raise(self._lib.agemm_check(self._h), "agemm_check")

    def close(self):
        if getattr(self, "_h", None):
            if getattr(self, "_pair", None) is not None:
                import torch
                torch.cuda.synchronize()
                self._pair = None
            self._lib.agemm_destroy(self._h)
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
