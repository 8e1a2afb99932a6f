"""Host checks of bench.py's command line (CPU only, no GPU touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_decode_bytes_of_the_four_shapes():
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    total = sum(bench.decode_bytes(s.K, s.N) for s in workloads.DECODE_SHAPES)
    assert total == 10975248          # packed W + bf16 X + fp32 Y + gamma, four shapes
