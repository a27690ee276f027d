"""GPU checks of the tiled population layout (lbm_params.tile_log2).

The layout changes where populations live, never what is computed, so a run
with tiles must give the fields of the same run stored one plane per
population bit for bit (that run is checked against the oracle by the other
parity tests).  Forced small tiles (64 and 512 cells) make every box here span
many tiles with a ragged last one, and put tile boundaries inside rows and
across walls, solids and open faces; forced tiles of 2^14 cells, the size
chosen automatically for isothermal fp32 boxes, leave a box of this size in
one or a few tiles with a ragged tail.  Thermal boxes keep their temperature
planes in the flow planes' tiles.  Automatic tiling is checked where it
engages at these sizes (fp64).  Submissions of 7 and 93 steps cover both step
parities and the graph replays."""
import numpy as np
import pytest

from harness import fluid_mask, gpu_run, oracle_run, say
from lattice_boltzmann_cfd_amd import binding, inputs
from test_gpu_2d import channel as channel2d
from test_gpu_2d import disks as disks2d
from test_gpu_faces import mixed_box
from test_gpu_parity import check_fields, dirichlet_spheres_case

pytestmark = pytest.mark.gpu


def ragged():
    w = inputs.sol128(shape=(70, 37, 23))
    w.params["accel"] = [2e-6, -1e-6, 5e-7]
    return w


CASES = {
    "ragged": ragged,
    "cavity": lambda: inputs.cavity256(shape=(34, 30, 26)),
    "spheres": dirichlet_spheres_case,
    "mixed_faces": mixed_box,
    "disks2d": disks2d,
    "channel2d": channel2d,
}


def same_fields(a, b, w, label):
    fl = fluid_mask(w)
    for k in ("rho", "u", "T"):
        if a[k] is None:
            continue
        x, y = a[k][..., fl], b[k][..., fl]
        assert np.array_equal(x, y), f"{label}: {k} differs by {np.abs(x - y).max():.3e}"


@pytest.mark.parametrize("dtype", [4, 8])
@pytest.mark.parametrize("tile", [6, 9, 14, 0])
@pytest.mark.parametrize("case", sorted(CASES))
def test_tiled_equals_untiled_bitwise(case, tile, dtype):
    say(f"CASE tiles {case} tile_log2={tile} dtype={dtype}")
    w = CASES[case]()
    w.params["tile_log2"] = 31
    ref = gpu_run(w, [7, 93], dtype=dtype)
    w.params["tile_log2"] = tile
    got = gpu_run(w, [7, 93], dtype=dtype)
    same_fields(got, ref, w, f"{case} tile_log2={tile}")
    for f_got, f_ref in zip(got["forces"], ref["forces"]):
        # the same link values, summed in a fixed order
        assert np.array_equal(f_got, f_ref)


@pytest.mark.parametrize("streaming,links", [(binding.LBM_STREAM_AB, binding.LBM_LINKS_IN_KERNEL),
                                             (binding.LBM_STREAM_AA, binding.LBM_LINKS_PASSES),
                                             (binding.LBM_STREAM_AB, binding.LBM_LINKS_PASSES),
                                             (binding.LBM_STREAM_AB_PUSH, binding.LBM_LINKS_IN_KERNEL)])
@pytest.mark.parametrize("case", ["spheres", "cavity", "disks2d"])
def test_tiled_two_buffer_and_link_passes(case, streaming, links):
    say(f"CASE tiles {case} streaming={streaming} links={links}")
    w = CASES[case]()
    w.params["links"] = links
    w.params["tile_log2"] = 31
    ref = gpu_run(w, [7, 93], streaming=streaming)
    w.params["tile_log2"] = 7
    got = gpu_run(w, [7, 93], streaming=streaming)
    same_fields(got, ref, w, f"{case} streaming={streaming} links={links}")


def test_tiled_against_the_oracle():
    """One tiled run straight against the oracle, with the parity bar."""
    say("CASE tiles vs oracle, thermal spheres, tile_log2=6, fp32")
    w = dirichlet_spheres_case()
    w.params["tile_log2"] = 6
    g = gpu_run(w, [100], dtype=4)
    o = oracle_run(w, 100)
    check_fields(g, o, w, 4, "tiles-oracle")
