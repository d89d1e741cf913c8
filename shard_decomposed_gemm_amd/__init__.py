"""Flag-gated, shard-decomposed AG+GEMM for one MI355X (gfx950).

The compute path is the HIP library libagemm.so (C-ABI in include/agemm.h
and, for the Flash-Decode combine, include/fdcombine.h); ``agemm`` and
``fdc`` are its ctypes bindings.
"""
from .agemm import AgemmError, Context, load, make_schedule, status_string  # noqa: F401
from .fdc import FdCombine  # noqa: F401
