"""CPU checks of bench.py's contract pieces that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True)
    assert out.returncode == 2
    assert "one GPU" in json.loads(out.stdout.strip())["error"]


def test_traffic_only_for_matching_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic("packed_text_32k") is None
    v = bench.measured_traffic("packed_multimodal_64k")
    # either the committed summary matches the current forward sources, or it is
    # stale and reported as unknown
    assert v is None or v > 1e8
