"""bench.py's command line on the host: more than one GPU is refused with a
message and exit status 2, and without a GPU the run fails loudly (no CPU
fallback that could print a throughput line)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_no_gpu_fails_loudly():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _bench("--quick", "--no-cpu-baseline", "--steps", "2", "--warmup", "1")
    assert r.returncode != 0
    assert '"metric"' not in r.stdout
