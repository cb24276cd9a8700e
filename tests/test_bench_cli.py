"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a JSON message and exit status 2."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_cache_flush_reads_its_buffer():
    """The cold-run flush (a read of its whole buffer) runs as written: here on
    the CPU with a small buffer."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    f = bench.CacheFlush(torch, torch.device("cpu"), nbytes=4096)
    f()
    assert float(f.out) == 1024.0
