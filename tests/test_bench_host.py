"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the
algorithmic byte counts of a RowNorm step, and which counter summaries the
JSON line may report."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_rownorm_step_bytes_by_kernel_class():
    # 18 B per element with bf16 gradients wherever the single pass takes
    # the matrix: read G 2, M 4, W 4; write M 4, W 4.
    wide, tall, too_tall, odd = (512, 2048), (4096, 1024), (40000, 256), (3000, 1001)
    b = bench.rownorm_class_bytes([wide, tall, too_tall, odd], 2)
    assert b["rownorm_rows"] == 18 * 512 * 2048
    assert b["rownorm_tall"] == 18 * 4096 * 1024
    # matrices the single pass does not take: G, M -> M, then M, W -> W
    two = 40000 * 256 + 3000 * 1001
    assert b["rownorm_cols1"] == 10 * two and b["rownorm_cols2"] == 12 * two
    # with the single pass off every tall matrix takes the two passes
    b2 = bench.rownorm_class_bytes([tall], 4, single_pass=False)
    assert b2.get("rownorm_tall", 0) == 0
    assert b2["rownorm_cols1"] == 12 * 4096 * 1024 and b2["rownorm_cols2"] == 12 * 4096 * 1024


def test_ns5_flops_of_one_square_matrix():
    # r = c = 4, 5 rounds: Gram (upper triangle) r^2 c, A^2 r^3, product 2 r^2 c
    f = bench.ns5_class_flops([(4, 4)])
    assert f == {"ns_gram": 5 * 64, "ns_poly": 5 * 64, "ns_product": 4 * 128, "ns_product_last": 128}
    # tall and wide matrices of the same sides count alike
    assert bench.ns5_class_flops([(8, 2)]) == bench.ns5_class_flops([(2, 8)])


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "ns_product_wl_hbm_traffic.txt"
    path.write_text("# a summary\n# source_sha256: not this one\nsource_sha256: abc\n"
                    "kernel: ns_product\ntraffic_bytes_per_launch: 1.5e+10\n")
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    return path


def test_traffic_is_reported_only_for_the_profiled_source(traffic_file, monkeypatch):
    monkeypatch.setattr(bench, "source_digest", lambda kernel: "abc")
    assert bench.measured_traffic("ns_product", "wl", True) == 1.5e10
    # another NS5 precision or workspace cap than the profiled run
    assert bench.measured_traffic("ns_product", "wl", False) is None
    # no summary for this workload
    assert bench.measured_traffic("ns_product", "other", True) is None
    # the kernel source changed since the counters were taken
    monkeypatch.setattr(bench, "source_digest", lambda kernel: "def")
    assert bench.measured_traffic("ns_product", "wl", True) is None


def test_source_digest_follows_the_kernel_file():
    # each kernel family is keyed by its own source file (and the shared header)
    d_ns, d_rn = bench.source_digest("ns_product"), bench.source_digest("rownorm_tall")
    assert d_ns == bench.source_digest("ns_gram") and d_ns != d_rn
    assert len(d_ns) == 64 and int(d_ns, 16) >= 0
