"""CPU checks of the C ABI (no device work): the library loads, exports every
function include/lbm.h declares, validates its arguments before touching the
device, and its host link builder finds exactly the blocked links."""
import os
import re

import numpy as np
import pytest

from lattice_boltzmann_cfd_amd import binding, inputs
from lattice_boltzmann_cfd_amd import build as lbm_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        lbm_build.build()
    return binding.library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lbm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lbm_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.ABI_FUNCTIONS)


def test_struct_layout_matches_header():
    # offsets implied by the header's field order and natural alignment
    P = binding.LbmParams
    assert P.face_T.offset == 72
    assert P.solid_T.offset == 128
    assert P.s19.offset == 136
    assert P.T0.offset == 136 + 8 * (19 + 7 + 1 + 3 + 3)
    assert P.face_u.offset == P.T0.offset + 8
    assert P.face_rho.offset == P.face_u.offset + 8 * 18
    assert P.lattice.offset == P.face_rho.offset + 8 * 6
    assert P.s9.offset == P.lattice.offset + 8
    assert P.s5.offset == P.s9.offset + 8 * 9
    assert P.tile_log2.offset == P.s5.offset + 8 * 5
    assert P.occupancy.offset == P.tile_log2.offset + 8
    assert binding.ctypes.sizeof(P) == P.occupancy.offset + 8


def periodic(n=8, **kw):
    return inputs.base_params(n, n, n, inputs.mrt_rates(0.6), **kw)


def test_required_bytes_sizes(lib):
    p = periodic(16)
    b4 = binding.lbm_required_bytes(p, dtype=4)
    b8 = binding.lbm_required_bytes(p, dtype=8)
    assert b4 >= 19 * 16 ** 3 * 4 and b8 >= 19 * 16 ** 3 * 8
    ab = binding.lbm_required_bytes(p, dtype=4, streaming=binding.LBM_STREAM_AB)
    assert ab >= 2 * 19 * 16 ** 3 * 4
    pt = dict(p, thermal=1, s7=[0, 1, 1, 1, 1, 1, 1])
    assert binding.lbm_required_bytes(pt) >= 26 * 16 ** 3 * 4


@pytest.mark.parametrize("mutate", [
    lambda p: p.update(nx=0),
    lambda p: p.update(face_kind=[1, 0, 0, 0, 0, 0]),
    lambda p: p.__setitem__("s19", [2.5] + p["s19"][1:]),
    lambda p: p.__setitem__("s19", p["s19"][:5] + [-0.1] + p["s19"][6:]),
    lambda p: p.update(a_T=-6.0),
    lambda p: p.update(accel=[float("nan"), 0, 0]),
    lambda p: p.update(face_thermal=[2, 0, 0, 0, 0, 0]),
    lambda p: p.update(face_kind=[5, 5, 0, 0, 0, 0]),
    lambda p: p.update(face_kind=[2, 0, 0, 0, 0, 0]),  # one face of x periodic, the other not
    lambda p: p.update(face_kind=[4, 4, 0, 0, 0, 0], face_rho=[0.0] * 6),
    lambda p: p.update(face_kind=[3, 1, 0, 0, 0, 0], face_u=[float("inf")] + [0.0] * 17),
    lambda p: p.update(face_kind=[2, 2, 0, 0, 0, 0], links=binding.LBM_LINKS_PASSES),
    lambda p: p.update(tile_log2=5),
    lambda p: p.update(tile_log2=21),
    lambda p: p.update(tile_log2=-1),
    lambda p: p.update(occupancy=[9, 0]),
    lambda p: p.update(occupancy=[0, -2]),
])
def test_invalid_params_rejected_without_device_work(lib, mutate):
    p = periodic()
    mutate(p)
    assert binding.lbm_required_bytes(p) == 0
    # a fake device pointer: any device access would fail with LBM_E_DEVICE
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, None, 256, 1 << 30)
    assert e.value.status == binding.LBM_E_INVALID


def test_bad_dtype_and_streaming(lib):
    p = periodic()
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, None, 256, 1 << 30, dtype=2)
    assert e.value.status == binding.LBM_E_INVALID
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, None, 256, 1 << 30, streaming=7)
    assert e.value.status == binding.LBM_E_INVALID


def test_push_streaming_needs_links_in_the_kernel(lib):
    """The one-pass two-buffer mode needs the two-pass mode's buffers and
    applies the boundary rules itself: link passes are rejected with it."""
    p = periodic(8, face_kind=[0, 0, 1, 1, 0, 0])
    push = binding.lbm_required_bytes(p, streaming=binding.LBM_STREAM_AB_PUSH)
    assert push == binding.lbm_required_bytes(p, streaming=binding.LBM_STREAM_AB) > 0
    q = dict(p, links=binding.LBM_LINKS_PASSES)
    assert binding.lbm_required_bytes(q, streaming=binding.LBM_STREAM_AB) > 0
    assert binding.lbm_required_bytes(q, streaming=binding.LBM_STREAM_AB_PUSH) == 0
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(q, None, 256, 1 << 30, streaming=binding.LBM_STREAM_AB_PUSH)
    assert e.value.status == binding.LBM_E_INVALID


def test_too_small_buffer_is_nomem(lib):
    p = periodic()
    need = binding.lbm_required_bytes(p)
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, None, 256, need - 1)
    assert e.value.status == binding.LBM_E_NOMEM


def test_null_context_calls_are_invalid(lib):
    out = (binding.ctypes.c_double * 16)()
    assert lib.lbm_init_fields(None, None, None, None) == binding.LBM_E_INVALID
    assert lib.lbm_step(None, 1) == binding.LBM_E_INVALID
    assert lib.lbm_read_macros(None, None, None, None) == binding.LBM_E_INVALID
    assert lib.lbm_wall_force(None, out, 4) == binding.LBM_E_INVALID
    assert lib.lbm_diagnostics(None, out, binding.LBM_DIAG_COUNT) == binding.LBM_E_INVALID
    assert lib.lbm_time(None) == -1
    assert lib.lbm_resume(None, 5) == binding.LBM_E_INVALID
    assert lib.lbm_num_links(None, 19) == -1
    assert lib.lbm_profile(None, 1) == binding.LBM_E_INVALID
    assert lib.lbm_profile_read(None, None, None, 0) == binding.LBM_E_INVALID
    lib.lbm_destroy(None)  # ignored


def test_solid_on_a_slip_layer_rejected(lib):
    n = 8
    p = periodic(n, face_kind=[0, 0, 2, 2, 0, 0])
    lab = np.zeros(n ** 3, np.uint8)
    lab[3 + n * 2 + n * n * 4] = 1  # y = 2: allowed
    assert binding.lbm_required_bytes(p, lab) > 0
    lab[5 + n * (n - 1) + n * n * 1] = 1  # y = n - 1: on the y+ slip layer
    assert binding.lbm_required_bytes(p, lab) == 0
    assert binding.lbm_count_links(p, lab, 19) == -1
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, lab, 256, 1 << 30)
    assert e.value.status == binding.LBM_E_INVALID


@pytest.mark.parametrize("face", range(6))
def test_solid_on_each_slip_layer_rejected(lib, face):
    """On a 6x7x5 box with the two faces of one axis SLIP: a solid cell one
    layer inside is accepted, one on the face's own layer is rejected."""
    shape = (6, 7, 5)
    a = face // 2
    kinds = [0] * 6
    kinds[2 * a] = kinds[2 * a + 1] = 2
    p = inputs.base_params(*shape, inputs.mrt_rates(0.6), face_kind=kinds)
    layer = shape[a] - 1 if face & 1 else 0
    inner = shape[a] - 2 if face & 1 else 1
    for pos, accepted in ((inner, True), (layer, False)):
        c = [3, 4, 2]
        c[a] = pos
        lab = np.zeros(shape[::-1], np.uint8)
        lab[c[2], c[1], c[0]] = 1
        lab = lab.reshape(-1)
        assert (binding.lbm_required_bytes(p, lab) > 0) == accepted, (face, pos)


@pytest.mark.parametrize("kinds", [[2] * 6, [3, 4, 2, 2, 1, 3], [4] * 6])
def test_link_counts_do_not_depend_on_face_kind(lib, kinds):
    """Every non-periodic face blocks the same links whatever its rule."""
    n = 6
    walls = inputs.base_params(n, n, n, inputs.mrt_rates(0.6), face_kind=[1] * 6, thermal=True,
                               s7=[0, 1, 1, 1, 1, 1, 1])
    other = dict(walls, face_kind=kinds)
    for lattice in (19, 7):
        assert binding.lbm_count_links(other, None, lattice) == binding.lbm_count_links(walls, None, lattice)


def test_box_too_large_rejected(lib):
    # a population plane is addressed with 32-bit byte offsets: 2^30 fp32 cells are too many
    p = inputs.base_params(2048, 1024, 512, inputs.mrt_rates(0.6))
    assert binding.lbm_required_bytes(p) == 0
    p = inputs.base_params(1024, 1024, 512, inputs.mrt_rates(0.6))
    assert binding.lbm_required_bytes(p) >= 19 * 4 * 2 ** 29


@pytest.mark.parametrize("shape,thermal,lattice", [((256, 256, 256), False, 0), ((70, 37, 23), True, 0),
                                                   ((512, 512, 512), True, 0), ((8193, 8193, 1), True, 1)])
def test_population_bytes_within_one_tile_of_the_minimum(lib, shape, thermal, lattice):
    """The tiled population layout wastes at most one partial tile (plus the
    plane shift of untiled boxes) per plane."""
    nx, ny, nz = shape
    if lattice:
        p = inputs.base_params_2d(nx, ny, inputs.mrt_rates_2d(0.6), thermal=thermal, s5=[0, 1, 1, 1, 1])
        q = 9 + (5 if thermal else 0)
    else:
        p = inputs.base_params(nx, ny, nz, inputs.mrt_rates(0.6), thermal=thermal, s7=[0, 1, 1, 1, 1, 1, 1])
        q = 19 + (7 if thermal else 0)
    b = binding.lbm_required_bytes(p, dtype=4)
    n = nx * ny * nz
    assert q * n * 4 <= b <= q * (n + 16384 + 1088) * 4 + (1 << 20)


@pytest.mark.parametrize("n", [1, 2, 5, 16])
def test_cavity_link_counts_closed_form(lib, n):
    """All-wall box: D3Q19 links = sum over directions of cells whose neighbour
    leaves the box = 6 n^2 (axis) + 12 n (2n - 1) (face diagonals);
    D3Q7 links = 6 n^2."""
    p = inputs.base_params(n, n, n, inputs.mrt_rates(0.6), face_kind=[1] * 6, thermal=True,
                           s7=[0, 1, 1, 1, 1, 1, 1])
    assert binding.lbm_count_links(p, None, 19) == 6 * n * n + 12 * n * (2 * n - 1)
    assert binding.lbm_count_links(p, None, 7) == 6 * n * n


def brute_force_links(p, lab, vel):
    nx, ny, nz = p["nx"], p["ny"], p["nz"]
    L = lab.reshape(nz, ny, nx)
    count = 0
    for c in vel:
        if not any(c):
            continue
        shifted = np.roll(L, shift=(-c[2], -c[1], -c[0]), axis=(0, 1, 2))  # label at x + c
        block = shifted != 0
        z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
        for a, (co, n) in enumerate(zip((x, y, z), (nx, ny, nz))):
            if p["face_kind"][2 * a]:
                block |= (co + c[a] < 0) | (co + c[a] >= n)
        count += int(np.count_nonzero(block & (L == 0)))
    return count


D3Q19 = [(0, 0, 0)] + [(a, b, c) for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)
                       if 0 < a * a + b * b + c * c <= 2]
D3Q7 = [(0, 0, 0), (1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0), (0, 0, 1), (0, 0, -1)]


@pytest.mark.parametrize("case", ["sphere_periodic", "spheres_walls"])
def test_solid_link_counts_brute_force(lib, case):
    if case == "sphere_periodic":
        n = 24
        lab = inputs.sphere_labels(n, n, n, 5.0)
        p = inputs.base_params(n, n, n, inputs.mrt_rates(0.6))
    else:
        lab, _ = inputs.random_spheres(30, 26, 22, rmin=2, rmax=4, fraction=0.1, seed=3)
        p = inputs.base_params(30, 26, 22, inputs.mrt_rates(0.6), face_kind=[0, 0, 0, 0, 1, 1])
    assert binding.lbm_count_links(p, lab, 19) == brute_force_links(p, lab, D3Q19)
    assert binding.lbm_count_links(p, lab, 7) == brute_force_links(p, lab, D3Q7)
    assert binding.lbm_required_bytes(p, lab) > binding.lbm_required_bytes(p, None)


# ------------------------------------------------------------ 2D variant

def square(n=8, **kw):
    return inputs.base_params_2d(n, n, inputs.mrt_rates_2d(0.6), **kw)


@pytest.mark.parametrize("mutate", [
    lambda p: p.update(nz=2),
    lambda p: p.update(face_kind=[0, 0, 0, 0, 1, 1]),
    lambda p: p.update(lattice=2),
    lambda p: p.__setitem__("s9", [2.5] + p["s9"][1:]),
    lambda p: p.__setitem__("s5", [0.0, -0.1, 1.0, 1.0, 1.0]),
    lambda p: p.update(a_T=-4.0),
    lambda p: p.update(accel=[0.0, 0.0, 1e-5]),
    lambda p: p.update(gbeta=[0.0, 0.0, 1e-5]),
    lambda p: p.update(face_kind=[3, 3, 0, 0, 0, 0], face_u=[0, 0, 1e-3] + [0.0] * 15),
])
def test_invalid_2d_params_rejected(lib, mutate):
    p = square()
    assert binding.lbm_required_bytes(p) > 0
    mutate(p)
    assert binding.lbm_required_bytes(p) == 0
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_create(p, None, 256, 1 << 30)
    assert e.value.status == binding.LBM_E_INVALID


def test_2d_sizes_and_lattice_numbers(lib):
    n = 64
    p = square(n, thermal=True, s5=[0, 1, 1, 1, 1])
    b = binding.lbm_required_bytes(p, dtype=8)
    assert 14 * n * n * 8 <= b < 19 * n * n * 8  # 9 + 5 planes, not 19 + 7
    # a 2D box has D2Q9 / D2Q5 link lists only
    assert binding.lbm_count_links(p, None, 19) == -1 and binding.lbm_count_links(p, None, 7) == -1
    assert binding.lbm_count_links(p, None, 9) == 0 and binding.lbm_count_links(p, None, 5) == 0


@pytest.mark.parametrize("n", [1, 2, 5, 16])
def test_square_cavity_link_counts_closed_form(lib, n):
    """All-wall square: D2Q9 links = 4 n (axis) + 4 (2n - 1) (diagonals);
    D2Q5 links = 4 n."""
    p = square(n, face_kind=[1] * 4, thermal=True, s5=[0, 1, 1, 1, 1])
    assert binding.lbm_count_links(p, None, 9) == 4 * n + 4 * (2 * n - 1)
    assert binding.lbm_count_links(p, None, 5) == 4 * n


D2Q9 = [(a, b, 0) for a in (-1, 0, 1) for b in (-1, 0, 1)]
D2Q5 = [(0, 0, 0), (1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0)]


def test_2d_solid_link_counts_brute_force(lib):
    nx, ny = 40, 31
    lab = inputs.sphere_labels(nx, ny, 1, 6.0, centre=(12.0, 15.5, 0.5))
    lab |= inputs.sphere_labels(nx, ny, 1, 4.0, centre=(38.0, 2.0, 0.5), label=2)  # wraps through x and y
    p = inputs.base_params_2d(nx, ny, inputs.mrt_rates_2d(0.6), face_kind=[0, 0, 1, 1], thermal=True,
                              s5=[0, 1, 1, 1, 1])
    assert binding.lbm_count_links(p, lab, 9) == brute_force_links(p, lab, D2Q9)
    assert binding.lbm_count_links(p, lab, 5) == brute_force_links(p, lab, D2Q5)


def test_tile_layout_buffer_sizes(lib):
    """On a box that is a whole number of tiles, tiles (any size; the thermal
    planes sharing the flow planes' tiles) need exactly the population bytes,
    while one plane per population adds the 1024-element plane shift to each
    of the 26 planes; the link arrays are the same for every layout."""
    w = inputs.cavity256(shape=(64, 64, 64))
    sizes = {}
    for d in (4, 8):
        for tile in (31, 13, 9, 6, 0):
            w.params["tile_log2"] = tile
            sizes[tile, d] = binding.lbm_required_bytes(w.params, None, dtype=d)
        for tile in (13, 9, 6, 0):
            assert abs((sizes[31, d] - sizes[tile, d]) - 26 * 1024 * d) <= 2 * 256, (tile, d)


@pytest.mark.parametrize("bad", ["short", "long", "negative", "too_large"])
def test_label_arrays_checked_by_the_binding(lib, bad):
    """The library reads nx*ny*nz label bytes; the binding refuses arrays of
    another size or values outside 0..255 before any call."""
    w = inputs.sphere128(shape=(12, 10, 8), R=3.0)
    lab = w.labels.astype(np.int64)
    if bad == "short":
        lab = lab[:-1]
    elif bad == "long":
        lab = np.concatenate([lab, [0]])
    elif bad == "negative":
        lab[5] = -1
    else:
        lab[5] = 256
    with pytest.raises(binding.LbmError) as e:
        binding.lbm_required_bytes(w.params, lab)
    assert e.value.status == binding.LBM_E_INVALID
    with pytest.raises(binding.LbmError):
        binding.lbm_count_links(w.params, lab, 19)
    # the same labels in range and of the right size are accepted, whatever their integer type
    assert binding.lbm_required_bytes(w.params, w.labels.astype(np.int32)) == binding.lbm_required_bytes(w.params, w.labels)


@pytest.mark.parametrize("shape,thermal,lattice,dtype,tiled", [
    ((512, 512, 512), True, 0, 4, True),    # D3Q19 + D3Q7 fp32, 14 GB: tiled
    ((512, 512, 512), False, 0, 4, False),  # D3Q19 fp32, 10 GB: one plane per population
    ((512, 512, 512), True, 0, 8, True),    # D3Q19 + D3Q7 fp64, 28 GB: tiled
    ((550, 550, 550), True, 0, 8, False),   # the same, 2^32 elements or more: one plane per population
    ((8193, 8193, 1), True, 1, 8, True),    # D2Q9 + D2Q5 fp64, 7.5 GB: tiled
    ((256, 256, 256), False, 0, 8, True),   # below 4 GiB: tiled whatever the kernel
    ((1021, 1030, 1020), False, 0, 4, False),  # 2^32 elements or more: one plane per population
])
def test_automatic_layout_of_large_buffers(lib, shape, thermal, lattice, dtype, tiled):
    """Buffers of 4 GiB or more are tiled only for the kernels measured faster
    that way (thermal 3D, thermal fp64 2D) and only below 2^32 elements;
    the rest keep one plane per population (the layout tile_log2 = 31 asks for)."""
    nx, ny, nz = shape
    if lattice:
        p = inputs.base_params_2d(nx, ny, inputs.mrt_rates_2d(0.6), thermal=thermal, s5=[0, 1, 1, 1, 1])
    else:
        p = inputs.base_params(nx, ny, nz, inputs.mrt_rates(0.6), thermal=thermal, s7=[0, 1, 1, 1, 1, 1, 1])
    auto = binding.lbm_required_bytes(p, dtype=dtype)
    planes = binding.lbm_required_bytes(dict(p, tile_log2=31), dtype=dtype)
    assert auto > 0 and planes > 0
    assert (auto != planes) == tiled


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library every call raises; nothing falls back to a
    CPU path."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "liblbm_hip.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        binding.lbm_required_bytes(periodic())
    with pytest.raises(RuntimeError, match="not built"):
        binding.lbm_check_links(periodic())
