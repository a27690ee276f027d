"""fp64 CPU oracle of the fused lattice Boltzmann time step (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``lattice_boltzmann_cfd_amd``) never does and has no CPU fallback.

The arithmetic lives in ``lbm_oracle.c`` (plain C, fp64, no blocking or
fusion); this module only compiles it with gcc, loads it with ctypes and
marshals numpy arrays.  See the header of ``lbm_oracle.c`` for the passages of
the pages each step follows and the readings taken where they are silent.
"""
from .oracle import (  # noqa: F401
    OracleParams,
    build,
    collide,
    equilibrium,
    library_path,
    run,
    lattice_sizes,
    tables,
    tables_2d,
    to_params,
)
