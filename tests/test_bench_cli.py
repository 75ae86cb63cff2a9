"""bench.py's command line on the host: more than one GPU is refused with a
message (the benchmark measures one GPU), before any GPU work."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                           text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, (n, r.returncode, r.stderr[-500:])
        msg = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in msg["error"]
