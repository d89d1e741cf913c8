"""bench.py's host side, without a GPU: the workloads' shapes, the roofline's
algorithmic work and bytes, the traffic lookup and the one-GPU refusal.

The expected flops and bytes are the closed forms 2MKN and 2KN + 6MK + c·MN
(B read once; A read by the producer, written to the inbox and read by the
consumer; C written once) evaluated by hand for each shape.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

# workload: (W, M, K, N, C bytes, 2MKN, path bytes)
SHAPES = {
    "tiny_m8": (8, 8, 512, 256, 4, 2_097_152, 294_912),
    "decode_m1": (8, 1, 8192, 28672, 2, 469_762_048, 469_868_544),
    "xover_m128": (8, 128, 8192, 28672, 2, 60_129_542_144, 483_393_536),
    "ooo_m512": (8, 512, 8192, 28672, 2, 240_518_168_576, 524_288_000),
    "prefill_m4096": (8, 4096, 8192, 28672, 2, 1_924_145_348_608, 905_969_664),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_workload_shapes_and_algorithmic_figures(name):
    W, M, K, N, cb, flops, path = SHAPES[name]
    w = bench.WORKLOADS[name]
    assert w[:4] == (W, M, K, N)
    assert w[4] == ("f32" if cb == 4 else "f16")
    f, consumer, p = bench.algorithmic(W, M, K, N, cb)
    assert f == flops
    assert p == path
    assert consumer == path - 4 * M * K  # the consumer alone reads A once and B once


def test_only_the_out_of_order_workload_has_a_release_schedule():
    assert {k for k, v in bench.WORKLOADS.items() if v[5]} == {"ooo_m512"}


def test_default_workload_is_the_largest_configuration():
    ap_default = [a for a in open(os.path.join(ROOT, "bench.py")).read().splitlines() if '"--workload"' in a]
    assert ap_default and 'default="prefill_m4096"' in ap_default[0]
    assert max(bench.WORKLOADS.values(), key=lambda v: v[1] * v[2] * v[3])[1] == 4096


def test_traffic_is_none_for_an_unknown_workload():
    assert bench.measured_traffic("no_such_workload", "mfma") is None


def test_kernel_digest_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; } // one\n/* two */\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ("k.hip",))
    d0 = bench.kernel_digest("probe")
    src.write_text("int f() {\n  return 1;  // another comment\n}\n")
    assert bench.kernel_digest("probe") == d0
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_digest("probe") != d0


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
