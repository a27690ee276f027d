"""lbm_step_noalloc against lbm_step, through the C ABI.

lbm_step_noalloc runs the same kernels with the step's scratch (gathered link
values, force-pass segment sums) in the library's static per-GPU array and
every kernel launched directly.  Its results must equal lbm_step's bit for
bit: fields, latched forces and heat, volume diagnostics.  Two cases run in a
row on one GPU, the second on a smaller box, so the second meets whatever the
first left in the shared array; each case covers link passes (the gathered
values live in the array) and bounce-back inside the step kernel (only the
segment sums do).  A context whose scratch would not fit is refused."""
import numpy as np
import pytest

from harness import say
from lattice_boltzmann_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu


def thermal_box(shape, links, seed):
    w = inputs.rb512(shape=shape, rmin=2, rmax=3, seed=seed)
    w.params["accel"] = [1e-5, -2e-6, 0.0]
    w.params["links"] = links
    return w


def run(w, steps, noalloc, dtype=4):
    import torch

    s = binding.Solver(w.params, w.labels, dtype=dtype)
    try:
        s.init(w.rho, w.u, w.T)
        forces = []
        for n in steps:
            (s.step_noalloc if noalloc else s.step)(n)
            forces.append(s.wall_force())
        rho, u, T = s.macros()
        diag = s.diagnostics()
        torch.cuda.synchronize()
        return dict(rho=rho.cpu().numpy(), u=u.cpu().numpy(), T=T.cpu().numpy(), forces=np.array(forces),
                    diag=diag)
    finally:
        s.close()


def same(a, b, what):
    for k in ("rho", "u", "T", "forces"):
        assert np.array_equal(a[k], b[k], equal_nan=True), f"{what}: {k}"
    # the volume sums add in an order set by atomics: equal to fp64 rounding
    assert np.allclose(a["diag"], b["diag"], rtol=1e-12, atol=1e-12), what


@pytest.mark.parametrize("dtype", [4, 8])
def test_noalloc_equals_step_two_calls_in_a_row(dtype):
    for shape, seed, steps in (((40, 36, 30), 7, [37, 18]), ((17, 13, 11), 8, [9, 4])):
        for links in (binding.LBM_LINKS_PASSES, binding.LBM_LINKS_IN_KERNEL):
            say(f"CASE noalloc shape={shape} links={links} dtype={dtype} steps={steps}")
            w = thermal_box(shape, links, seed)
            ref = run(w, steps, False, dtype)
            got = run(w, steps, True, dtype)
            same(got, ref, f"{shape} links={links}")
            assert np.abs(ref["forces"][-1]).max() > 0


def test_noalloc_refuses_a_context_whose_scratch_does_not_fit():
    import torch

    # a 3D checkerboard of solid cells: every fluid cell has its six axis
    # neighbours solid, so 6 flow and 6 temperature links per fluid cell
    n = 72
    i = np.arange(n ** 3)
    x, y, z = i % n, (i // n) % n, i // (n * n)
    lab = ((x + y + z) % 2).astype(np.uint8)
    p = inputs.base_params(n, n, n, inputs.mrt_rates(0.6), thermal=True, s7=inputs.thermal_rates(0.05))
    p["links"] = binding.LBM_LINKS_PASSES
    nl = binding.lbm_count_links(p, lab, 19) + binding.lbm_count_links(p, lab, 7)
    assert 8 * nl > binding.LBM_NOALLOC_SCRATCH_BYTES
    say(f"CASE noalloc refusal: {nl} links in fp64")
    s = binding.Solver(p, lab, dtype=8)
    try:
        rho, u, T = inputs.rest(n, n, n)
        s.init(rho, u, T)
        with pytest.raises(binding.LbmError, match="scratch"):
            s.step_noalloc(2)
        s.step(2)  # the context itself is fine
        torch.cuda.synchronize()
    finally:
        s.close()
