"""The C++ link builder's own run-time check (host only, through the C ABI).

lbm_check_links builds the links lbm_create would build and checks what the
in-place scheme relies on: no two links store into one slot, in the
bounce-back inside the step kernel and in the link passes after even and odd
steps, and every solid cell leaves the slot a fluid neighbour bounces into to
that neighbour (its mask bit).  lbm_create runs the same check before it
uploads anything.  Every box kind the library accepts must pass: the
degenerate boxes (one cell, one cell thick between walls, every cell a
corner, a fluid cell caged by solids, a one-cell gap between slip faces, a
one-cell channel from inlet to outlet, the 2D single cell and strip), the
box recipes of the measured workloads at small sizes, slip and open faces,
and both link modes and streaming modes.  The tests/test_aa_scheme_cpu.py
models check the same property on a Python re-model of the builder."""
import numpy as np
import pytest

from lattice_boltzmann_cfd_amd import binding, inputs
from test_aa_faces_cpu import case as face_case
from test_aa_faces_cpu import degenerate_face_case
from test_aa_scheme_cpu import case as scheme_case
from test_aa_scheme_cpu import degenerate_case

PER, WALL, SLIP, VEL, PRES = (inputs.FACE_PERIODIC, inputs.FACE_WALL, inputs.FACE_SLIP, inputs.FACE_VELOCITY,
                              inputs.FACE_PRESSURE)


def modes(p, lab):
    """(params, streaming) of every link mode and streaming mode the box allows."""
    open_faces = any(k in (SLIP, VEL, PRES) for k in p["face_kind"])
    out = []
    for streaming in (binding.LBM_STREAM_AA, binding.LBM_STREAM_AB, binding.LBM_STREAM_AB_PUSH):
        out.append((dict(p, links=binding.LBM_LINKS_IN_KERNEL), streaming))
        if not open_faces and streaming != binding.LBM_STREAM_AB_PUSH:
            out.append((dict(p, links=binding.LBM_LINKS_PASSES), streaming))
    return out


def check_all(p, lab):
    for q, streaming in modes(p, lab):
        binding.lbm_check_links(q, lab, streaming=streaming)


@pytest.mark.parametrize("name", ["one_cell", "one_thick_gap", "corners", "caged_cell"])
def test_degenerate_boxes(name):
    p, lab, _, _, _ = degenerate_case(name)
    check_all(p, lab)


@pytest.mark.parametrize("name", ["slip_gap", "open_rod"])
def test_degenerate_face_boxes(name):
    p, lab, _, _, _ = degenerate_face_case(name)
    check_all(p, lab)


@pytest.mark.parametrize("name", ["walls_solids", "cavity_thermal", "rb_spheres", "dirichlet_solid"])
def test_wall_and_solid_boxes(name):
    p, lab, _, _, _ = scheme_case(name)
    check_all(p, lab)


@pytest.mark.parametrize("name", ["slip_sphere", "lid", "inlet_outlet_thermal", "mixed_edges"])
def test_face_rule_boxes(name):
    p, lab, _, _, _ = face_case(name)
    check_all(p, lab)


@pytest.mark.parametrize("name,shape,kw", [("rb512", (48, 40, 36), {}), ("cavity256", (20, 18, 16), {}),
                                           ("sphere128", (32, 32, 32), {}), ("channel256", (40, 24, 24), {"R": 5.0}),
                                           ("cavity2d", (33, 29), {})])
def test_workload_recipes(name, shape, kw):
    w = inputs.make(name, shape=shape, **kw)
    check_all(w.params, w.labels)


@pytest.mark.parametrize("nx,ny", [(1, 1), (1, 7), (9, 1), (6, 5)])
def test_2d_boxes_with_walls_and_solids(nx, ny):
    p = inputs.base_params_2d(nx, ny, inputs.mrt_rates_2d(0.6), thermal=True, face_kind=[WALL, WALL, SLIP, SLIP]
                              if nx > 1 and ny > 2 else [WALL, WALL, PER, PER], face_thermal=[1, 1, 0, 0],
                              face_T=[0.5, -0.5, 0, 0], s5=inputs.thermal_rates_2d(0.05))
    lab = np.zeros(nx * ny, np.uint8)
    if nx >= 5 and ny >= 5:
        lab[2 + nx * 2] = 3  # a solid cell away from the slip layers
    check_all(p, lab if lab.any() else None)


def test_rejected_parameters_are_reported():
    p = inputs.base_params(4, 4, 4, inputs.mrt_rates(0.6), face_kind=[SLIP, SLIP, PER, PER, PER, PER])
    lab = np.zeros(64, np.uint8)
    lab[0] = 1  # a solid cell in the first layer of the x- slip face
    with pytest.raises(binding.LbmError, match="SLIP"):
        binding.lbm_check_links(p, lab)
    with pytest.raises(binding.LbmError):
        binding.lbm_check_links(dict(p, nx=0))
