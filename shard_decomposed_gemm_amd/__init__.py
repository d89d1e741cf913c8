"""Flag-gated, shard-decomposed AG+GEMM for one MI355X (gfx950).

The compute path is the HIP library libagemm.so (C-ABI in include/agemm.h);
``agemm`` is its ctypes binding.
"""
from .agemm import AgemmError, Context, load, make_schedule, status_string  # noqa: F401
