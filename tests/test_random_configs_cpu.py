"""Host checks of the link builder on the seeded random configurations of the
GPU sweep (no device work): for every drawn box, the number of links
lbm_count_links reports per lattice equals a brute-force count of the blocked
(fluid cell, direction) pairs (the neighbour x + c leaves through a bounded
face or is a solid cell), and lbm_check_links finds no slot stored twice, in
the drawn streaming and link mode."""
import numpy as np
import pytest

from lattice_boltzmann_cfd_amd import binding
from test_abi import brute_force_links
from test_gpu_random_configs import N_CASES, draw

D3Q19 = [(0, 0, 0)] + [(a, b, c) for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)
                       if 0 < a * a + b * b + c * c <= 2]
D3Q7 = [(0, 0, 0), (1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0), (0, 0, 1), (0, 0, -1)]
D2Q9 = [(a, b, 0) for a in (-1, 0, 1) for b in (-1, 0, 1)]
D2Q5 = [(0, 0, 0), (1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0)]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_link_counts_and_check(seed):
    w, dtype, streaming, _, _ = draw(seed)
    p = w.params
    lab = w.labels if w.labels is not None else np.zeros(w.cells, np.uint8)
    two_d = int(p.get("lattice", 0)) == 1
    lattices = [(9, D2Q9), (5, D2Q5)] if two_d else [(19, D3Q19), (7, D3Q7)]
    for code, vel in lattices[:2 if p["thermal"] else 1]:
        assert binding.lbm_count_links(p, w.labels, code) == brute_force_links(p, lab, vel), (seed, code)
    binding.lbm_check_links(p, w.labels, dtype, streaming)
