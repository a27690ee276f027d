"""The workloads at their own lengths, in fp32, with what must hold over the
whole run (stability at the low-viscosity rates of the thermal boxes is the
risk: tau = 0.5205 in the 256^3 cavity, 0.5129 in the 512^3 cell).

  * 128^3 solenoidal box, 1000 steps: finite, mass and momentum of the
    periodic box kept to fp32 rounding, and in-place, two-buffer and one-pass
    two-buffer streaming equal bit for bit after 1000 steps;
  * 128^3 sphere under a body force, 2000 steps, drag read every 100 steps:
    the drag grows from rest and stays below the total body force (the fluid
    is still accelerating);
  * 256^3 heated cavity, 5000 steps: finite, closed-box mass kept, heat
    enters through the hot wall and leaves through the cold one;
  * 512^3 random-sphere convection cell, 1000 steps: the same;
  * 385^3 heated cavity (the thermal page's 3D grid and length), 6000 steps:
    the same.
Each run is repeated in fp64 (the build the oracle pins at 1e-11) and the
largest fp32 - fp64 field differences at the end are printed: they are the
drift of fp32 rounding over the run.  Measured on MI355X (fp32 mass change
over the run; largest fp32 - fp64 field difference at the end):
  sol128    1000 steps   1.3e-10   6.2e-8 (rho), 1.1e-8 (u)
  sphere128 2000 steps   2.9e-10   6.0e-8 (rho), 7.1e-10 (u); drag 1.3e-7 rel.
  cavity256 5000 steps   1.6e-11   6.2e-8 (rho), 8.8e-9 (u), 9.0e-8 (T)
  rb512     1000 steps   1.1e-8    6.0e-8 (rho), 5.3e-11 (u), 1.5e-7 (T)
  cavity385 6000 steps   6.2e-12   6.2e-8 (rho), 8.0e-9 (u), 1.0e-7 (T)
The bounds are about a hundred times these; a population lost or doubled at
one cell each step would change the mass by about steps / cells (6e-3 at
128^3 after 1000 steps, 7e-6 at 512^3)."""
import numpy as np
import pytest

from harness import fluid_mask, say
from lattice_boltzmann_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu


def run(w, submissions, dtype, streaming=binding.LBM_STREAM_AUTO, read_force=False):
    import torch

    thermal = bool(w.params.get("thermal"))
    s = binding.Solver(w.params, w.labels, dtype=dtype, streaming=streaming)
    try:
        s.init(w.rho, w.u, w.T if thermal else None)
        d0 = s.diagnostics()
        forces = []
        for n in submissions:
            s.step(n)
            if read_force:
                forces.append(s.wall_force())
        d1 = s.diagnostics()  # raises LBM_E_UNSTABLE if a fluid value is not finite
        rho, u, T = s.macros()
        torch.cuda.synchronize()
        out = dict(d0=d0, d1=d1, forces=forces, rho=rho.cpu().double().numpy(), u=u.cpu().double().numpy(),
                   T=T.cpu().double().numpy() if T is not None else None, heat=s.wall_force()[:, 3])
        return out
    finally:
        s.close()
        torch.cuda.empty_cache()


def drift(a, b, fl):
    d = {"rho": np.abs(a["rho"][fl] - b["rho"][fl]).max(), "u": np.abs(a["u"][:, fl] - b["u"][:, fl]).max()}
    if a["T"] is not None:
        d["T"] = np.abs(a["T"][fl] - b["T"][fl]).max()
    return d


def mass_change(r):
    return abs(r["d1"][binding.LBM_DIAG_MASS] - r["d0"][binding.LBM_DIAG_MASS]) / r["d0"][binding.LBM_DIAG_MASS]


def test_sol128_1000_steps():
    w = inputs.make("sol128")
    say("CASE sol128, 1000 steps, fp32 in place / two buffers / one pass, and fp64")
    runs = {m: run(w, [1000], 4, m) for m in (binding.LBM_STREAM_AA, binding.LBM_STREAM_AB,
                                              binding.LBM_STREAM_AB_PUSH)}
    aa = runs[binding.LBM_STREAM_AA]
    for m, r in runs.items():
        assert np.array_equal(r["rho"], aa["rho"]) and np.array_equal(r["u"], aa["u"]), m
    d64 = run(w, [1000], 8)
    fl = fluid_mask(w)
    dm = mass_change(aa)
    mom = np.abs(aa["d1"][2:5] - aa["d0"][2:5]).max() / w.cells
    say(f"  fp32 mass change {dm:.3e}, momentum change per cell {mom:.3e}, umax {aa['d1'][6]:.4f}; "
        f"fp32-fp64 drift {drift(aa, d64, fl)}; fp64 mass change {mass_change(d64):.3e}")
    assert np.isfinite(aa["u"]).all()
    assert dm <= 1e-8
    assert mass_change(d64) <= 1e-13
    assert mom <= 1e-9
    assert max(drift(aa, d64, fl).values()) <= 1e-5


def test_sphere128_2000_steps_drag_every_100():
    w = inputs.make("sphere128")
    say("CASE sphere128, 2000 steps, drag every 100, fp32 and fp64")
    r32 = run(w, [100] * 20, 4, read_force=True)
    r64 = run(w, [100] * 20, 8, read_force=True)
    fl = fluid_mask(w)
    drag32 = np.array([f[6, 0] for f in r32["forces"]])
    drag64 = np.array([f[6, 0] for f in r64["forces"]])
    total = w.params["accel"][0] * r32["d1"][binding.LBM_DIAG_MASS]  # body force on the fluid per step
    say(f"  drag every 100 steps (fp32): {np.array2string(drag32, precision=4)}; total body force {total:.4e}")
    say(f"  fp32-fp64 drag rel diff {np.abs(drag32 - drag64).max() / drag64.max():.3e}; "
        f"field drift {drift(r32, r64, fl)}; fp32 mass change {mass_change(r32):.3e}")
    assert (drag32 > 0).all()
    assert drag32[-1] > drag32[9] > drag32[0]
    assert (drag32 < total).all()
    assert np.abs(drag32 - drag64).max() <= 1e-5 * drag64.max()
    assert max(drift(r32, r64, fl).values()) <= 1e-5
    assert mass_change(r32) <= 1e-8


def thermal_case(name, w, steps, mass_tol):
    say(f"CASE {name}, {steps} steps, fp32 and fp64")
    r32 = run(w, [steps], 4)
    r64 = run(w, [steps], 8)
    fl = fluid_mask(w)
    axis = 0 if name in ("cavity256", "cavity385") else 2
    hot, cold = r32["heat"][2 * axis], r32["heat"][2 * axis + 1]
    say(f"  fp32: mass change {mass_change(r32):.3e}, umax {r32['d1'][binding.LBM_DIAG_UMAX]:.4f}, "
        f"Q hot {hot:.4e}, Q cold {cold:.4e}; fp64 mass change {mass_change(r64):.3e}, "
        f"Q hot {r64['heat'][2 * axis]:.4e}; fp32-fp64 drift {drift(r32, r64, fl)}")
    assert np.isfinite(r32["u"][:, fl]).all() and np.isfinite(r32["T"][fl]).all()
    assert hot > 0 > cold
    assert mass_change(r32) <= mass_tol
    assert mass_change(r64) <= 1e-12
    assert max(drift(r32, r64, fl).values()) <= 1e-5


def test_cavity256_5000_steps():
    thermal_case("cavity256", inputs.make("cavity256"), 5000, 1e-9)


def test_rb512_1000_steps():
    thermal_case("rb512", inputs.make("rb512"), 1000, 1e-6)


def test_cavity385_6000_steps():
    """The thermal page's 3D grid and length (385^3, 6000 steps, run in double
    precision there), with the heated-cavity recipe; fp32 against fp64 as
    above."""
    thermal_case("cavity385", inputs.make("cavity385"), 6000, 1e-9)
