"""The oracle, and the measurement arithmetic, against values the pages print
(tests/golden/, each file citing its page and section)."""
import os

import numpy as np
import pytest

import bench
import oracle
from lattice_boltzmann_cfd_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].split()
            if line:
                yield line


@pytest.mark.parametrize("row", list(rows("abb_constants.txt")), ids=lambda r: f"{r[0]}-aT{r[1]}")
def test_antibounceback_constant_is_twice_the_moving_weight(row):
    """The oracle's equilibrium at rest, T = 0.37: every moving temperature
    population is omega T / 2 with the page's omega."""
    lattice, a_T, omega = row[0], float(row[1]), float(row[2])
    if lattice == "D3Q7":
        p = dict(nx=1, ny=1, nz=1, thermal=1, s19=[1.0] * 19, s7=[1.0] * 7, a_T=a_T)
    else:
        p = inputs.base_params_2d(1, 1, [1.0] * 9, thermal=True, s5=[1.0] * 5, a_T=a_T)
    T = 0.37
    _, geq = oracle.equilibrium(p, np.array([1.0]), np.zeros((1, 3)), np.array([T]))
    moving = geq[0][1:]
    assert len(moving) == (6 if lattice == "D3Q7" else 4)
    assert np.allclose(2 * moving, omega * T, rtol=0, atol=1e-15)


@pytest.mark.parametrize("row", [r for r in rows("bytes_per_update.txt") if r[0] == "layout"], ids=lambda r: r[1])
def test_bytes_per_update_of_the_two_layouts(row):
    """The bench's algorithmic bytes per cell update equal the page's 152 B
    (in place) and 304 B (two buffers, two passes) for D3Q19 in fp32."""
    values, per_value = int(row[2]), int(row[3])
    streaming = 1 if row[1].startswith("aa") else 2
    assert bench.bytes_per_cell(False, 4, streaming) == values * per_value


@pytest.mark.parametrize("row", [r for r in rows("bytes_per_update.txt") if r[0] == "bound"], ids=lambda r: r[1])
def test_bandwidth_bound_and_fraction(row):
    """The bench's conversions between cell updates and HBM bytes reproduce
    the page's bounds and roofline fractions from its own inputs."""
    values, per_value, gbps = int(row[2]), int(row[3]), float(row[4])
    bound, measured, frac = float(row[5]), float(row[6]), float(row[7])
    bpu = values * per_value
    assert round(bench.mlups_at(gbps, bpu), 1) == bound
    assert round(100 * bench.hbm_gbps(measured, bpu) / gbps, 1) == frac
