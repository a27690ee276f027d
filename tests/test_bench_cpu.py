"""Host-side parts of bench.py (no GPU): the one-GPU guard and the CPU
baseline leg's record."""
import os
import subprocess
import sys

import bench
from lattice_boltzmann_cfd_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_record():
    w = inputs.tg32(shape=(16, 12, 10))
    rec = bench.cpu_baseline(w, 2, 1)
    assert rec["unit"] == "MLUPS" and rec["kind"] == "oracle"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "16x12x10" in rec["sample"]
    one = rec["one_thread"]
    assert one["cores"] == 1 and one["value"] > 0
    assert bench.cpu_baseline(w, 1, 0).get("one_thread") is None
