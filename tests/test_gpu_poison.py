"""GPU check that the kernels write no population slot that no cell owns.

lbm_create sets every byte of the population buffers (plane padding, the tail
of the last tile, the second buffer of the two-buffer modes) and of the link
scratch to 0xff, a NaN in either precision; lbm_init_fields writes the slots
the cells own (solid cells get the canonical NaN, whose bit pattern differs).
After that, the set of 32-bit words that still read 0xffffffff must not
change over any number of steps: a store into a slot no cell owns, or a
padding NaN copied into an owned slot, would change it.  In place with the
boundary rules inside the step kernel, nothing but owned slots is written
from the first step on; the two-buffer modes write their second buffer in
the first step and the link passes their scratch, so for them the set is
compared from the second step on.  The fluid fields stay finite throughout
(a padding NaN read by a fluid cell would show there).  Boxes with ragged
tiles, one plane per population (with its plane shift), walls, solids, open
faces and the 2D lattices, in both precisions."""
import numpy as np
import pytest

from harness import fluid_mask, say
from lattice_boltzmann_cfd_amd import binding
from test_gpu_tiles import CASES

pytestmark = pytest.mark.gpu

AA, AB, PUSH = binding.LBM_STREAM_AA, binding.LBM_STREAM_AB, binding.LBM_STREAM_AB_PUSH

RUNS = [
    ("ragged", 31, AA, 0), ("ragged", 6, AA, 0), ("ragged", 0, PUSH, 0), ("ragged", 9, AB, 0),
    ("cavity", 31, AA, 0), ("cavity", 9, AA, 0), ("cavity", 9, AB, 0), ("cavity", 6, AA, 1),
    ("spheres", 31, AA, 0), ("spheres", 6, AA, 0), ("spheres", 9, PUSH, 0), ("spheres", 9, AA, 1),
    ("mixed_faces", 31, AA, 0), ("mixed_faces", 9, AA, 0),
    ("disks2d", 31, AA, 0), ("disks2d", 6, AA, 1), ("channel2d", 9, AA, 0),
]


def all_ones(torch, buf):
    """Which 32-bit words of the device buffer read 0xffffffff."""
    return (buf.view(torch.int32) == -1).cpu().numpy()


@pytest.mark.parametrize("dtype", [4, 8])
@pytest.mark.parametrize("case,tile,streaming,passes", RUNS)
def test_unowned_slots_stay_untouched(case, tile, streaming, passes, dtype):
    import torch

    say(f"CASE poison {case} tile_log2={tile} streaming={streaming} passes={passes} dtype={dtype}")
    w = CASES[case]()
    w.params["tile_log2"] = tile
    w.params["links"] = binding.LBM_LINKS_PASSES if passes else binding.LBM_LINKS_IN_KERNEL
    thermal = bool(w.params.get("thermal"))
    s = binding.Solver(w.params, w.labels, dtype=dtype, streaming=streaming)
    try:
        s.init(w.rho, w.u, w.T if thermal else None)
        s.stream.synchronize()
        sets = {0: all_ones(torch, s.buf)}
        t = 0
        for n in (2, 5, 93):
            s.step(n)
            s.stream.synchronize()
            t += n
            sets[t] = all_ones(torch, s.buf)
        rho, u, T = s.macros()
        torch.cuda.synchronize()
        fl = fluid_mask(w)
        assert np.isfinite(rho.cpu().numpy()[fl]).all() and np.isfinite(u.cpu().numpy()[:, fl]).all()
        if T is not None:
            assert np.isfinite(T.cpu().numpy()[fl]).all()
        s.wall_force()  # raises LBM_E_UNSTABLE if a read-back saw a non-finite fluid value
    finally:
        s.close()
    counts = {k: int(v.sum()) for k, v in sets.items()}
    say(f"  words reading 0xffffffff after 0, 2, 7, 100 steps: {list(counts.values())}")
    assert counts[2] > 0
    first = 0 if (streaming == AA and not passes) else 2
    for k in (2, 7, 100):
        if k > first:
            changed = np.flatnonzero(sets[first] != sets[k])
            assert changed.size == 0, f"{changed.size} words changed between steps {first} and {k}, first {changed[:8]}"
