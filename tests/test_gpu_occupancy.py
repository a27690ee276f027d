"""GPU checks of lbm_params.occupancy (resident blocks per compute unit).

A bound on the blocks that share a compute unit changes when blocks run,
never what a block computes, so every bound must give the fields of the
unbounded run bit for bit (that run is checked against the oracle by the other
parity tests).  Bounds of 1 block (a reservation above 64 KiB of local data
share, which raises the kernel's limit first), 2 and 3, different for even and
odd steps, on boxes with walls, solids, open faces and both lattices;
submissions of 7 and 93 steps cover both parities and the graph replays."""
import numpy as np
import pytest

from harness import gpu_run, say
from lattice_boltzmann_cfd_amd import binding
from test_gpu_tiles import CASES, same_fields

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("occ", [(1, 2), (3, -1), (-1, 1)])
@pytest.mark.parametrize("dtype", [4, 8])
@pytest.mark.parametrize("case", sorted(CASES))
def test_bounded_occupancy_equals_unbounded_bitwise(case, dtype, occ):
    say(f"CASE occupancy {case} dtype={dtype} occupancy={occ}")
    w = CASES[case]()
    w.params["occupancy"] = [-1, -1]
    ref = gpu_run(w, [7, 93], dtype=dtype)
    w.params["occupancy"] = list(occ)
    got = gpu_run(w, [7, 93], dtype=dtype)
    same_fields(got, ref, w, f"{case} occupancy={occ}")
    for f_got, f_ref in zip(got["forces"], ref["forces"]):
        # the same link values, summed in a fixed order
        assert np.array_equal(f_got, f_ref)


@pytest.mark.parametrize("streaming", [binding.LBM_STREAM_AB, binding.LBM_STREAM_AB_PUSH])
@pytest.mark.parametrize("case", ["spheres", "disks2d"])
def test_bounded_occupancy_two_buffers(case, streaming):
    say(f"CASE occupancy two buffers {case} streaming={streaming}")
    w = CASES[case]()
    w.params["occupancy"] = [-1, -1]
    ref = gpu_run(w, [7, 93], streaming=streaming)
    w.params["occupancy"] = [2, 1]
    got = gpu_run(w, [7, 93], streaming=streaming)
    same_fields(got, ref, w, f"{case} two buffers, streaming {streaming}")
