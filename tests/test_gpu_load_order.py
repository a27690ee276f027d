"""The binding works whatever the caller touches first.

torch ships its own HIP runtime under the system runtime's soname.  When the
library was loaded before torch (a host-only call such as lbm_required_bytes
made first), the process held two runtimes and the library's found no
device: every lbm_create failed with LBM_E_DEVICE.  The binding now imports
torch before it loads the library.  This runs, in a fresh process, a host-only
call first, then a solver, and checks its fields after 10 steps against the
same run in this process."""
import os
import subprocess
import sys

import numpy as np
import pytest

from harness import gpu_run, say
from lattice_boltzmann_cfd_amd import inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
from lattice_boltzmann_cfd_amd import binding, inputs
w = inputs.tg32()
assert binding.lbm_required_bytes(w.params) > 0  # the library's first call, before any torch call here
import torch
s = binding.Solver(w.params, None)
s.init(w.rho, w.u)
s.step(10)
rho, u, T = s.macros()
torch.cuda.synchronize()
np.save(sys.argv[2], np.concatenate([rho.cpu().double().numpy(), u.cpu().double().numpy().reshape(-1)]))
s.close()
"""


def test_host_call_before_torch(tmp_path):
    say("CASE binding: a host-only call first, in a fresh process, then a solver")
    out = str(tmp_path / "fields.npy")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, out], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    child = np.load(out)
    g = gpu_run(inputs.tg32(), [10], want_forces=False)
    assert np.array_equal(child, np.concatenate([g["rho"], g["u"].reshape(-1)]))
