"""The C-ABI library loads, exports every function include/agemm.h declares,
and rejects bad shapes before touching the GPU. No compute calls here."""
import ctypes
import os
import re

import pytest

from shard_decomposed_gemm_amd import agemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "agemm.h")


HEADER_FD = os.path.join(ROOT, "include", "fdcombine.h")


def _declared(header=HEADER, prefix="agemm_"):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(" + prefix + r"[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_documented_entry_points():
    names = _declared()
    for must in ("agemm_create", "agemm_produce", "agemm_run_fused", "agemm_run_bsp"):
        assert must in names
    assert sorted(agemm.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = agemm.load()
    for name in _declared() + _declared(HEADER_FD, "fdc_"):
        assert hasattr(lib, name), name


def test_fd_header_matches_binding():
    from shard_decomposed_gemm_amd import fdc
    names = _declared(HEADER_FD, "fdc_")
    for must in ("fdc_create", "fdc_produce", "fdc_run_fused", "fdc_run_bsp"):
        assert must in names
    assert sorted(fdc.EXPORTED) == names
    fdc.load()  # every signature resolves


@pytest.mark.parametrize("W,H,D,HT,code", [
    (0, 96, 128, 16, agemm.ESHAPE),    # no ranks
    (17, 96, 128, 16, agemm.ESHAPE),   # too many ranks
    (8, 0, 128, 16, agemm.ESHAPE),     # no heads
    (8, 96, 96, 16, agemm.ESHAPE),     # D not 64, 128 or 256
    (8, 96, 128, 6, agemm.ESHAPE),     # heads per tile not a multiple of 4
    (8, 96, 128, 36, agemm.ESHAPE),    # heads per tile above 32
    (8, 100, 128, 16, agemm.ESHAPE),   # heads per tile does not divide H
    (8, 96, 128, 4, agemm.ESHAPE),     # T = 8 * 24 = 192 tiles, above 64
])
def test_fd_create_rejects_bad_shapes_without_gpu(W, H, D, HT, code):
    from shard_decomposed_gemm_amd import fdc
    lib = fdc.load()
    h = ctypes.c_void_p()
    assert lib.fdc_create(ctypes.byref(h), W, H, D, HT, agemm.F16) == code
    assert not h.value
    assert lib.fdc_create(ctypes.byref(h), 8, 96, 128, 16, 7) == agemm.EINVAL  # unknown dtype


def test_status_strings():
    assert agemm.status_string(0) == "AGEMM_OK"
    assert agemm.status_string(5) == "AGEMM_ETIMEOUT"
    assert agemm.status_string(99) == "AGEMM_UNKNOWN"


@pytest.mark.parametrize("W,M,K,N,code", [
    (0, 1, 512, 256, agemm.ESHAPE),     # no shards
    (17, 1, 17 * 64, 256, agemm.ESHAPE),  # too many shards
    (8, 0, 512, 256, agemm.ESHAPE),     # empty M
    (8, 1, 500, 256, agemm.ESHAPE),     # K not a multiple of W
    (8, 1, 8 * 96, 256, agemm.ESHAPE),  # K/W not a multiple of 64
    (8, 1, 512, 250, agemm.ESHAPE),     # N not a multiple of 8
    (8, 1, 512, 0, agemm.ESHAPE),
    (8, 1, (1 << 22) + 8 * 64, 256, agemm.ESHAPE),  # K past the 32-bit lane-offset bound
    (8, 1, 512, (1 << 24) + 8, agemm.ESHAPE),       # N past the 32-bit lane-offset bound
])
def test_create_rejects_bad_shapes_without_gpu(W, M, K, N, code):
    lib = agemm.load()
    h = ctypes.c_void_p()
    assert lib.agemm_create(ctypes.byref(h), W, M, K, N, agemm.F16, 0) == code
    assert not h.value


def test_create_rejects_bad_flag_tile_and_dtype():
    lib = agemm.load()
    h = ctypes.c_void_p()
    assert lib.agemm_create(ctypes.byref(h), 8, 4, 8192, 256, agemm.F16, 96) == agemm.ESHAPE   # not /64
    assert lib.agemm_create(ctypes.byref(h), 8, 4, 8192, 256, agemm.F16, 384) == agemm.ESHAPE  # does not divide 1024
    assert lib.agemm_create(ctypes.byref(h), 16, 4, 16 * 4096, 256, agemm.F16, 64) == agemm.ESHAPE  # T > 64
    assert lib.agemm_create(ctypes.byref(h), 8, 4, 8192, 256, 7, 0) == agemm.EINVAL
    assert lib.agemm_create(None, 8, 4, 8192, 256, agemm.F16, 0) == agemm.EINVAL


@pytest.mark.parametrize("value", ["4294967296", "-1", "0x1ffffffff", "12abc", ""])
def test_epoch_base_hook_refuses_values_it_cannot_take(value, monkeypatch):
    """AGEMM_EPOCH_BASE (the testing hook that starts the epoch counters near their wrap)
    is checked before anything is allocated: a value that is not a number in 0..2^32-1
    makes both context kinds return EINVAL, with no device involved."""
    lib = agemm.load()
    monkeypatch.setenv("AGEMM_EPOCH_BASE", value)
    h = ctypes.c_void_p()
    assert lib.agemm_create(ctypes.byref(h), 8, 4, 8192, 256, agemm.F16, 0) == agemm.EINVAL
    assert not h.value
    assert lib.fdc_create(ctypes.byref(h), 8, 96, 128, 16, agemm.F16) == agemm.EINVAL
    assert not h.value
    # a valid value passes the check: the shape check that follows still runs
    monkeypatch.setenv("AGEMM_EPOCH_BASE", str(2**32 - 3))
    assert lib.agemm_create(ctypes.byref(h), 8, 1, 512, 250, agemm.F16, 0) == agemm.ESHAPE


def test_null_context_is_rejected():
    lib = agemm.load()
    assert lib.agemm_run_fused(None, None, None, None) == agemm.EINVAL
    assert lib.agemm_produce(None, None, None, None) == agemm.EINVAL
    assert lib.agemm_check(None) == agemm.EINVAL
    assert lib.agemm_destroy(None) == agemm.OK
    assert lib.agemm_last_error(None) == b"no context"
    assert lib.agemm_set_order(None, 1) == agemm.EINVAL
    g, sp = ctypes.c_int32(), ctypes.c_int32()
    assert lib.agemm_consumer_grid(None, ctypes.byref(g), ctypes.byref(sp)) == agemm.EINVAL
    assert lib.agemm_consumer_kernel(None, None, None) == agemm.EINVAL


def test_probes_reject_bad_arguments_without_gpu():
    """The calibration probes validate their arguments before any HIP call."""
    lib = agemm.load()
    v = ctypes.c_double()
    i = ctypes.c_int32()
    assert lib.agemm_device_info(None, ctypes.byref(i), ctypes.byref(i), ctypes.byref(i)) == agemm.EINVAL
    assert lib.agemm_probe_mfma(1, 1, None, None, ctypes.byref(v)) == agemm.EINVAL      # no out buffer
    assert lib.agemm_probe_mfma(-1, 1, 64, None, ctypes.byref(v)) == agemm.EINVAL       # warmup < 0
    assert lib.agemm_probe_mfma(0, 0, 64, None, ctypes.byref(v)) == agemm.EINVAL        # no timed launch
    assert lib.agemm_probe_mfma(0, 1, 64, None, None) == agemm.EINVAL                   # no result pointer
    assert lib.agemm_probe_read(64, 15, 0, 1, 64, None, ctypes.byref(v)) == agemm.EINVAL  # not a multiple of 16
    assert lib.agemm_probe_read(72, 64, 0, 1, 64, None, ctypes.byref(v)) == agemm.EINVAL  # misaligned buffer
    assert lib.agemm_probe_read(None, 64, 0, 1, 64, None, ctypes.byref(v)) == agemm.EINVAL
    assert lib.agemm_probe_read(64, 64, 0, 1, 66, None, ctypes.byref(v)) == agemm.EINVAL  # misaligned out


def test_plain_c_program_links_and_calls_the_library(tmp_path):
    """The boundary is a C ABI: a C99 program that includes both headers links against
    libagemm.so and calls host-only entry points (no GPU needed): the work plan of the
    prefill workload, a status name, and a shape error from agemm_create."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = agemm.load()._name
    libdir = os.path.dirname(lib)
    src = tmp_path / "main.c"
    src.write_text(
        "#include <stdio.h>\n#include \"agemm.h\"\n#include \"fdcombine.h\"\n"
        "int main(void) {\n"
        "  int32_t cfg = -9, grid = -9, split = -9;\n"
        "  int rc = agemm_mfma_plan(4096, 28672, 8192, 8, 256, -1, -1, &cfg, &grid, &split);\n"
        "  printf(\"%s %d %d %d\\n\", agemm_status_string(rc), cfg, grid, split);\n"
        "  agemm_ctx* ctx = 0;\n"
        "  printf(\"%s\\n\", agemm_status_string(agemm_create(&ctx, 8, 4, 8192 + 8, 256, AGEMM_F16, 0)));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "main"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-L", libdir, "-lagemm", "-Wl,-rpath," + libdir,
                        "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split("\n")[:2] == ["AGEMM_OK 0 256 0", "AGEMM_ESHAPE"]
