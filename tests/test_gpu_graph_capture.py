"""lbm_step_noalloc under HIP graph capture, replayed.

lbm_step_noalloc launches every kernel directly on the context's stream and
allocates nothing, so a caller can capture it into a graph.  The graph holds
the launches of one call with that call's step parities; the context's time
(host state) advances once, at capture, so the caller captures an even
number of steps and sets the time with lbm_resume after replays.  Here a
2-step call is captured on the solver's stream, the graph is replayed four
times with the program's own eager work and synchronisations between the
replays (a read-back, torch arithmetic on it), and after every replay the
fields and the latched forces must equal an eager run of as many steps, bit
for bit.  Both link modes: bounce-back in the kernel (scratch: the force
pass's segment sums) and link passes (also the gathered link values)."""
import numpy as np
import pytest

from harness import say
from lattice_boltzmann_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu


def box(links):
    w = inputs.rb512(shape=(30, 26, 22), rmin=2, rmax=3, seed=11)
    w.params["accel"] = [1e-5, 0.0, -2e-6]
    w.params["links"] = links
    return w


def read(torch, s):
    rho, u, T = s.macros()
    torch.cuda.synchronize()
    return [x.cpu().double().numpy() for x in (rho, u, T)], s.wall_force()


@pytest.mark.parametrize("links", [binding.LBM_LINKS_IN_KERNEL, binding.LBM_LINKS_PASSES])
def test_noalloc_captured_and_replayed(links):
    import torch

    say(f"CASE graph capture of lbm_step_noalloc, links={links}")
    w = box(links)
    eager = binding.Solver(w.params, w.labels)
    side = torch.cuda.Stream()
    cap = binding.Solver(w.params, w.labels, stream=side)
    try:
        eager.init(w.rho, w.u, w.T)
        cap.init(w.rho, w.u, w.T)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            cap.step_noalloc(2)
        for k in range(1, 5):
            g.replay()
            torch.cuda.synchronize()
            binding.lbm_resume(cap.ctx, 2 * k)  # the time, which replays do not advance
            eager.step_noalloc(2)
            (f_cap, force_cap), (f_eager, force_eager) = read(torch, cap), read(torch, eager)
            for a, b in zip(f_cap, f_eager):
                assert np.array_equal(a, b, equal_nan=True), f"replay {k}: fields differ"
            assert np.array_equal(force_cap, force_eager), f"replay {k}: forces differ"
            # the program's own eager work between replays
            junk = torch.from_numpy(f_cap[0]).cuda().mul_(2.0).sum()
            torch.cuda.synchronize()
            del junk
            say(f"  replay {k}: t = {cap.time}, equal to {2 * k} eager steps")
    finally:
        cap.close()
        eager.close()
