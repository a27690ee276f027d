"""Pin of the oracle's window mode (CPU only).

The oracle can run on a window of the box: a sub-box that may wrap through
periodic faces.  Populations pulled from outside the window are NaN, so after
n steps a cell lies on the exact side of the NaN front when every cut edge of
the window (a window boundary that is not a box face) is more than n cells
away along its axis: the front moves at most one cell per step along each
axis.  The full-size parity tests of the GPU path compare against windows of
the large boxes, so the window code has to give the full-domain result bit
for bit on those cells.  Here each case runs the oracle on the whole box and
on windows of it (walls, solid spheres, open faces, the temperature lattice,
the 2D lattice pair, windows wrapping through periodic faces and windows
against walls) and compares every such cell.  The NaN fill itself is checked
as well: it must reach the cells next to a cut after one step, or the exact
region would be claimed on a wrong argument.
"""
import numpy as np
import pytest

import oracle
from lattice_boltzmann_cfd_amd import inputs

PER, WALL, SLIP, VEL, PRES = (inputs.FACE_PERIODIC, inputs.FACE_WALL, inputs.FACE_SLIP, inputs.FACE_VELOCITY,
                              inputs.FACE_PRESSURE)


def window_cells(shape, lo, wn):
    """Global indices of a window's cells in the window's own (local) order."""
    N = np.array(shape)
    k, j, i = np.meshgrid(np.arange(wn[2]), np.arange(wn[1]), np.arange(wn[0]), indexing="ij")
    gx = (lo[0] + i.reshape(-1)) % N[0]
    gy = (lo[1] + j.reshape(-1)) % N[1]
    gz = (lo[2] + k.reshape(-1)) % N[2]
    return gx + N[0] * (gy + N[1] * gz), (i.reshape(-1), j.reshape(-1), k.reshape(-1))


def exact_mask(shape, lo, wn, nonperiodic, steps):
    """Local cells that no NaN from a cut edge can reach in `steps` steps.

    Along an axis the window's low end is a cut unless it is the box's low
    face of a non-periodic axis (lo = 0); its high end likewise unless it is
    the high face.  A window spanning a periodic axis whole has no cut on it.
    """
    _, (i, j, k) = window_cells(shape, lo, wn)
    ok = np.ones(i.size, bool)
    for a, li in enumerate((i, j, k)):
        if wn[a] == shape[a]:
            continue
        low_cut = not (nonperiodic[a] and lo[a] == 0)
        high_cut = not (nonperiodic[a] and lo[a] + wn[a] == shape[a])
        if low_cut:
            ok &= li >= steps
        if high_cut:
            ok &= li <= wn[a] - 1 - steps
    return ok


def check_windows(p, labels, rho, u, T, steps, windows):
    shape = (p["nx"], p["ny"], p["nz"])
    full = oracle.run(p, steps, rho, u, T, labels=labels)
    nonper = [p["face_kind"][2 * a] != PER for a in range(3)]
    thermal = bool(p.get("thermal"))
    fluid = np.ones(np.prod(shape), bool) if labels is None else labels == 0
    for lo, wn in windows:
        gidx, _ = window_cells(shape, lo, wn)
        Tw = T[gidx] if thermal else None
        o = oracle.run(p, steps, rho[gidx], u[:, gidx], Tw, labels=labels, window=(lo, wn))
        ok = exact_mask(shape, lo, wn, nonper, steps) & fluid[gidx]
        assert ok.sum() >= 8, (lo, wn, ok.sum())
        g = gidx[ok]
        # bit for bit: the same operations in the same order on the same values
        assert np.array_equal(o["rho"][ok], full["rho"][g]), (lo, wn)
        assert np.array_equal(o["u"][:, ok], full["u"][:, g]), (lo, wn)
        if thermal:
            assert np.array_equal(o["T"][ok], full["T"][g]), (lo, wn)
        # no NaN survives in the exact region, and the front did start moving
        assert np.isfinite(o["rho"][ok]).all()
        one = oracle.run(p, 1, rho[gidx], u[:, gidx], Tw, labels=labels, window=(lo, wn))
        cut_near = ~exact_mask(shape, lo, wn, nonper, 1) & fluid[gidx]
        if cut_near.any():
            assert np.isnan(one["rho"][cut_near]).any(), (lo, wn)


def thermal_wall_box():
    """Thermal box: x walls (hot/cold Dirichlet), periodic y and z, two
    solid spheres (one Dirichlet label rule for all solids), buoyancy."""
    nx, ny, nz = 14, 16, 15
    lab = inputs.sphere_labels(nx, ny, nz, 2.2, centre=(5.0, 1.0, 5.5))          # crosses the y- face
    lab |= inputs.sphere_labels(nx, ny, nz, 1.8, centre=(10.0, 8.0, 14.5), label=2)  # crosses the z+ face
    p = inputs.base_params(nx, ny, nz, inputs.mrt_rates(0.62), thermal=True, s7=inputs.thermal_rates(0.08),
                           face_kind=[WALL, WALL, PER, PER, PER, PER], face_thermal=[1, 1, 0, 0, 0, 0],
                           face_T=[0.5, -0.5, 0, 0, 0, 0], gbeta=(0.0, 0.0, 2e-3), accel=(1e-5, 0.0, -2e-5),
                           solid_thermal=inputs.DIRICHLET, solid_T=0.2)
    rho, u = inputs.taylor_green(nx, ny, nz, u0=0.03, seed=21)
    T = 0.4 * np.random.default_rng(22).uniform(-1, 1, rho.size)
    return p, lab, rho, u, T


def open_face_box():
    """Velocity inlet x-, pressure outlet x+, slip y faces, walls z, a sphere."""
    nx, ny, nz = 16, 10, 9
    lab = inputs.sphere_labels(nx, ny, nz, 2.0, centre=(7.0, 5.0, 4.5))
    fu = np.zeros((6, 3))
    fu[0] = (0.03, 0.004, -0.002)
    fu[5] = (0.02, 0.0, 0.0)
    p = inputs.base_params(nx, ny, nz, inputs.mrt_rates(0.7), face_kind=[VEL, PRES, SLIP, SLIP, WALL, VEL],
                           face_u=fu, face_rho=[1.0, 0.996, 1, 1, 1, 1.01], accel=(1e-5, 0.0, 0.0))
    rho, u = inputs.taylor_green(nx, ny, nz, u0=0.02, seed=23)
    return p, lab, rho, u


@pytest.mark.parametrize("steps", [3, 5])
def test_window_equals_full_box_thermal_walls_and_solids(steps):
    p, lab, rho, u, T = thermal_wall_box()
    windows = [
        ((0, 12, 9), (14, 14, 13)),  # whole x (against both walls), wraps through the y and z faces
        ((2, 3, 0), (12, 16, 15)),   # cut on both x ends, y and z whole
        ((0, 0, 0), (14, 16, 15)),   # the whole box as a window
        ((0, 14, 3), (9, 16, 15)),   # against the x- wall, cut before x+, y whole from y = 14
    ]
    check_windows(p, lab, rho, u, T, steps, windows)


def test_window_equals_full_box_open_faces():
    p, lab, rho, u = open_face_box()
    windows = [
        ((0, 0, 0), (12, 10, 9)),   # against the inlet, cut before the outlet
        ((5, 0, 0), (11, 10, 9)),   # cut after the inlet, against the outlet (pressure rule, own velocity)
        ((3, 2, 1), (12, 8, 8)),    # cut on every axis, against the z+ lid
    ]
    check_windows(p, lab, rho, u, None, 4, windows)


def test_window_equals_full_box_periodic_wraps():
    nx, ny, nz = 13, 12, 14
    p = inputs.base_params(nx, ny, nz, inputs.mrt_rates(0.58), accel=(2e-5, -1e-5, 1e-5))
    rho, u = inputs.solenoidal(nx, ny, nz, umax=0.05, kmax=3, seed=24)
    windows = [((9, 7, 6), (12, 11, 13)), ((12, 0, 8), (13, 12, 14)), ((4, 5, 2), (11, 12, 11))]
    check_windows(p, None, rho, u, None, 4, windows)


def test_window_equals_full_box_2d_thermal():
    nx, ny = 30, 21
    s5 = inputs.thermal_rates_2d(0.05)
    p = inputs.base_params_2d(nx, ny, inputs.mrt_rates_2d(0.6), thermal=True, s5=s5,
                              face_kind=[PER, PER, WALL, WALL], face_thermal=[0, 0, 1, 1],
                              face_T=[0, 0, 0.5, -0.5], gbeta=(0.0, 2e-3))
    rho, u = inputs.taylor_green(nx, ny, 1, u0=0.03, seed=25)
    u[2] = 0.0
    T = 0.3 * np.random.default_rng(26).uniform(-1, 1, rho.size)
    windows = [((25, 0, 0), (20, 21, 1)), ((3, 4, 0), (22, 15, 1))]
    check_windows(p, None, rho, u, T, 5, windows)
