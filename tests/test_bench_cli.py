"""bench.py's contract on the CPU: more than one GPU is refused with a message
(the path is built for one GPU), and the algorithmic byte counts of the step
match the shapes of the workloads (what `value` divides by)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_is_for_the_dominant_op():
    sys.path.insert(0, ROOT)
    import json

    import bench

    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    T, H = 16384, 32768
    # read g and y, write dgrad (bf16), read the bias, write dbias (fp32)
    assert t["algorithmic_bytes_per_launch"] == T * H * 6 + H * 2 + H * 4
    assert t["bytes_per_launch"] >= t["algorithmic_bytes_per_launch"]
