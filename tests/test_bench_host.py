"""Host-side logic of bench.py that runs without a GPU: the one-GPU guard,
and the rule that a recorded HBM-traffic figure is reported only while the
kernel source it was measured on is unchanged."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_needs_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    digest = bench.source_digest("quantize.hip", "block_quant.h", "internal.h")
    (tmp_path / "quantize_w_traffic.md").write_text(
        f"# summary\n\nsource_digest: {digest}\ntraffic_bytes_per_launch: 2.79365e+07\n")
    assert bench.recorded_traffic("quantize", "w", digest) == 2.79365e7
    assert bench.recorded_traffic("quantize", "w", "0" * 16) is None      # source changed since
    assert bench.recorded_traffic("quantize", "other", digest) is None    # never measured


def test_source_digest_covers_every_named_file():
    a = bench.source_digest("gemm.hip", "gemm_large.hip", "internal.h")
    b = bench.source_digest("gemm.hip", "gemm_small.hip", "internal.h")
    assert a != b and len(a) == 16
