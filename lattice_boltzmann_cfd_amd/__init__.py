"""MI355X-native fused lattice Boltzmann time step.

The compute path is the C-ABI library ``liblbm_hip.so`` (hand-written HIP
kernels for gfx950) declared in ``include/lbm.h``; ``binding`` wraps it with
ctypes (argument marshalling only).  ``inputs`` makes the seeded synthetic
workloads.  The binding loads the library on first use and raises if it is
missing: there is no CPU fallback.
"""
from . import binding, inputs  # noqa: F401

__all__ = ["inputs", "binding"]
