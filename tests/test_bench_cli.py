"""bench.py's host-side contract: it measures one GPU and says so for more, and
it takes HBM traffic only from a counter summary taken on the current kernel
source."""
import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=e)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    r = run_bench("--gpus", "1", env={"WORLD_SIZE": "8"})
    assert r.returncode == 2


def test_traffic_only_from_a_summary_of_the_current_source(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// kernels\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    good = tmp_path / "good.md"
    good.write_text(f"kernel_source_sha256: {sha}\n\ntraffic_bytes_per_launch[w13+w2]: 1.5e+08\n")
    assert bench.kernel_traffic(str(good), "w13+w2", str(src)) == 1.5e8
    assert bench.kernel_traffic(str(good), "w13", str(src)) is None      # other kernel
    stale = tmp_path / "stale.md"
    stale.write_text("kernel_source_sha256: " + "0" * 64 + "\n\ntraffic_bytes_per_launch[w13+w2]: 1.5e+08\n")
    assert bench.kernel_traffic(str(stale), "w13+w2", str(src)) is None
    assert bench.kernel_traffic(str(tmp_path / "missing.md"), "w13+w2", str(src)) is None


def test_percentiles_and_cpu_model():
    p = bench.percentiles(list(range(101)))
    assert (p["p10"], p["p50"], p["p90"]) == (10.0, 50.0, 90.0)
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_algorithmic_bytes_per_expert():
    # 2-bit g128 gate/up of one expert at H=4096, I=2048: 4 MiB codes + 256 KiB scales
    assert bench.per_expert_bytes(2, 128, 4096, 4096) == 4 * 2 ** 20 + 256 * 2 ** 10
    assert bench.per_expert_bytes(2, 64, 4096, 2048) == 2 * 2 ** 20 + 256 * 2 ** 10
