"""ctypes binding of ``liblbm_hip.so`` (the C ABI declared in include/lbm.h).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  The library is loaded on first use; if it is missing or fails to
load, every call raises -- there is no CPU fallback.  PyTorch is used by
:class:`Solver` only to allocate device memory and to name the HIP stream.

Functions with the ABI's names take and return plain values: device pointers
as integers, the parameter dict of :mod:`lattice_boltzmann_cfd_amd.inputs`,
host arrays as numpy.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblbm_hip.so")

LBM_OK, LBM_E_INVALID, LBM_E_NOMEM, LBM_E_DEVICE, LBM_E_UNSTABLE = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "LBM_OK", 1: "LBM_E_INVALID", 2: "LBM_E_NOMEM", 3: "LBM_E_DEVICE", 4: "LBM_E_UNSTABLE"}
LBM_STREAM_AUTO, LBM_STREAM_AA, LBM_STREAM_AB, LBM_STREAM_AB_PUSH = 0, 1, 2, 3
LBM_LINKS_IN_KERNEL, LBM_LINKS_PASSES = 0, 1
LBM_LATTICE_3D, LBM_LATTICE_2D = 0, 1
LBM_FACE_PERIODIC, LBM_FACE_WALL, LBM_FACE_SLIP, LBM_FACE_VELOCITY, LBM_FACE_PRESSURE = 0, 1, 2, 3, 4
MAX_GROUPS = 261
(LBM_DIAG_FLUID_CELLS, LBM_DIAG_MASS, LBM_DIAG_MOM_X, LBM_DIAG_MOM_Y, LBM_DIAG_MOM_Z, LBM_DIAG_KINETIC,
 LBM_DIAG_UMAX, LBM_DIAG_HEAT, LBM_DIAG_CONV_X, LBM_DIAG_CONV_Y, LBM_DIAG_CONV_Z, LBM_DIAG_COUNT) = range(12)
(LBM_KERNEL_STEP_EVEN, LBM_KERNEL_STEP_ODD, LBM_KERNEL_AB_COLLIDE, LBM_KERNEL_AB_PULL, LBM_KERNEL_LINK_GATHER,
 LBM_KERNEL_LINK_SCATTER, LBM_KERNEL_LINK_DIRECT, LBM_KERNEL_FORCE, LBM_KERNEL_KINDS) = range(9)
KERNEL_NAMES = ("step_even", "step_odd", "ab_collide", "ab_pull", "link_gather", "link_scatter", "link_direct",
                "force")

# every function the header declares
ABI_FUNCTIONS = (
    "lbm_required_bytes", "lbm_create", "lbm_init_fields", "lbm_step", "lbm_read_macros",
    "lbm_wall_force", "lbm_diagnostics", "lbm_time", "lbm_resume", "lbm_num_links", "lbm_count_links", "lbm_last_error",
    "lbm_destroy", "lbm_profile", "lbm_profile_read", "lbm_check_links", "lbm_step_noalloc",
)
LBM_NOALLOC_SCRATCH_BYTES = 16 << 20


class LbmParams(ctypes.Structure):
    """Mirror of ``lbm_params`` in include/lbm.h."""

    _fields_ = [
        ("nx", ctypes.c_int32), ("ny", ctypes.c_int32), ("nz", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("streaming", ctypes.c_int32), ("thermal", ctypes.c_int32),
        ("face_kind", ctypes.c_int32 * 6), ("face_thermal", ctypes.c_int32 * 6),
        ("face_T", ctypes.c_double * 6),
        ("solid_thermal", ctypes.c_int32), ("links", ctypes.c_int32),
        ("solid_T", ctypes.c_double),
        ("s19", ctypes.c_double * 19), ("s7", ctypes.c_double * 7),
        ("a_T", ctypes.c_double), ("accel", ctypes.c_double * 3), ("gbeta", ctypes.c_double * 3),
        ("T0", ctypes.c_double),
        ("face_u", ctypes.c_double * 18), ("face_rho", ctypes.c_double * 6),
        ("lattice", ctypes.c_int32), ("pad1", ctypes.c_int32),
        ("s9", ctypes.c_double * 9), ("s5", ctypes.c_double * 5),
        ("tile_log2", ctypes.c_int32), ("pad2", ctypes.c_int32), ("occupancy", ctypes.c_int32 * 2),
    ]


class LbmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def library():
    """Load liblbm_hip.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m lattice_boltzmann_cfd_amd.build` "
                               "(there is no CPU fallback)")
        # torch ships its own HIP runtime under the system runtime's soname.
        # Loaded first, it is the copy this library binds to, and the process
        # holds one runtime.  Loaded after this library, it would bring a
        # second runtime beside the system one, and this library's would then
        # find no device.
        import torch  # noqa: F401

        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(LbmParams)
        vp = ctypes.c_void_p
        lib.lbm_required_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_uint8)]
        lib.lbm_required_bytes.restype = ctypes.c_size_t
        lib.lbm_create.argtypes = [P, ctypes.POINTER(ctypes.c_uint8), vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
        lib.lbm_create.restype = ctypes.c_int
        lib.lbm_init_fields.argtypes = [vp, vp, vp, vp]
        lib.lbm_init_fields.restype = ctypes.c_int
        lib.lbm_step.argtypes = [vp, ctypes.c_int64]
        lib.lbm_step.restype = ctypes.c_int
        lib.lbm_read_macros.argtypes = [vp, vp, vp, vp]
        lib.lbm_read_macros.restype = ctypes.c_int
        lib.lbm_wall_force.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.c_int32]
        lib.lbm_wall_force.restype = ctypes.c_int
        lib.lbm_diagnostics.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.c_int32]
        lib.lbm_diagnostics.restype = ctypes.c_int
        lib.lbm_time.argtypes = [vp]
        lib.lbm_time.restype = ctypes.c_int64
        lib.lbm_resume.argtypes = [vp, ctypes.c_int64]
        lib.lbm_resume.restype = ctypes.c_int
        lib.lbm_num_links.argtypes = [vp, ctypes.c_int32]
        lib.lbm_num_links.restype = ctypes.c_int64
        lib.lbm_count_links.argtypes = [P, ctypes.POINTER(ctypes.c_uint8), ctypes.c_int32]
        lib.lbm_count_links.restype = ctypes.c_int64
        lib.lbm_check_links.argtypes = [P, ctypes.POINTER(ctypes.c_uint8)]
        lib.lbm_check_links.restype = ctypes.c_int
        lib.lbm_step_noalloc.argtypes = [vp, ctypes.c_int64]
        lib.lbm_step_noalloc.restype = ctypes.c_int
        lib.lbm_last_error.argtypes = [vp]
        lib.lbm_last_error.restype = ctypes.c_char_p
        lib.lbm_destroy.argtypes = [vp]
        lib.lbm_destroy.restype = None
        lib.lbm_profile.argtypes = [vp, ctypes.c_int32]
        lib.lbm_profile.restype = ctypes.c_int
        lib.lbm_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int32]
        lib.lbm_profile_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def to_params(d: dict, dtype: int = 4, streaming: int = LBM_STREAM_AUTO) -> LbmParams:
    """Marshal the shared parameter dict into ``lbm_params``."""
    p = LbmParams()
    p.nx, p.ny, p.nz = int(d["nx"]), int(d["ny"]), int(d["nz"])
    p.dtype = int(dtype)
    p.streaming = int(streaming)
    p.thermal = int(d.get("thermal", 0))
    for i in range(6):
        p.face_kind[i] = int(d.get("face_kind", [0] * 6)[i])
        p.face_thermal[i] = int(d.get("face_thermal", [0] * 6)[i])
        p.face_T[i] = float(d.get("face_T", [0.0] * 6)[i])
    p.solid_thermal = int(d.get("solid_thermal", 0))
    p.links = int(d.get("links", LBM_LINKS_IN_KERNEL))
    p.solid_T = float(d.get("solid_T", 0.0))
    for i in range(19):
        p.s19[i] = float(d.get("s19", [0.0] * 19)[i])
    for i in range(7):
        p.s7[i] = float(d.get("s7", [0.0] * 7)[i])
    p.lattice = int(d.get("lattice", LBM_LATTICE_3D))
    for i in range(9):
        p.s9[i] = float(d.get("s9", [0.0] * 9)[i])
    for i in range(5):
        p.s5[i] = float(d.get("s5", [0.0] * 5)[i])
    p.tile_log2 = int(d.get("tile_log2", 0))
    occ = d.get("occupancy", (0, 0))
    p.occupancy[0], p.occupancy[1] = int(occ[0]), int(occ[1])
    p.a_T = float(d.get("a_T", 0.0))
    for i in range(3):
        p.accel[i] = float(d.get("accel", [0.0] * 3)[i])
        p.gbeta[i] = float(d.get("gbeta", [0.0] * 3)[i])
    p.T0 = float(d.get("T0", 0.0))
    fu = np.asarray(d.get("face_u", np.zeros(18)), dtype=float).reshape(-1)
    fr = d.get("face_rho", [1.0] * 6)
    for i in range(18):
        p.face_u[i] = float(fu[i])
    for i in range(6):
        p.face_rho[i] = float(fr[i])
    return p


def _labels_ptr(labels, params: dict):
    """Pointer to the labels as nx*ny*nz contiguous bytes (the library reads
    exactly that many); a label array of another size or with values outside
    0..255 is rejected here."""
    if labels is None:
        return ctypes.POINTER(ctypes.c_uint8)(), None
    src = np.asarray(labels)
    cells = int(params["nx"]) * int(params["ny"]) * int(params["nz"])
    if src.size != cells:
        raise LbmError(LBM_E_INVALID, f"solid labels hold {src.size} values, the box has {cells} cells")
    if src.dtype != np.uint8 and src.size and (src.min() < 0 or src.max() > 255):
        raise LbmError(LBM_E_INVALID, "solid labels must lie in 0..255")
    arr = np.ascontiguousarray(src, dtype=np.uint8).reshape(-1)
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), arr


def _check(ctx, status):
    if status != LBM_OK:
        raise LbmError(status, lbm_last_error(ctx))


def lbm_required_bytes(params: dict, labels=None, dtype=4, streaming=LBM_STREAM_AUTO) -> int:
    p = to_params(params, dtype, streaming)
    lp, _keep = _labels_ptr(labels, params)
    return int(library().lbm_required_bytes(ctypes.byref(p), lp))


def lbm_create(params: dict, labels, device_buf: int, device_bytes: int, stream: int = 0, dtype=4,
               streaming=LBM_STREAM_AUTO):
    """Returns the context handle (an integer)."""
    p = to_params(params, dtype, streaming)
    lp, _keep = _labels_ptr(labels, params)
    out = ctypes.c_void_p()
    st = library().lbm_create(ctypes.byref(p), lp, ctypes.c_void_p(device_buf), device_bytes,
                              ctypes.c_void_p(stream), ctypes.byref(out))
    if st != LBM_OK:
        raise LbmError(st, lbm_last_error(None))
    return out.value


def lbm_init_fields(ctx, rho: int, u: int, T: int | None = None):
    _check(ctx, library().lbm_init_fields(ctypes.c_void_p(ctx), ctypes.c_void_p(rho), ctypes.c_void_p(u),
                                          ctypes.c_void_p(T or 0)))


def lbm_step(ctx, n: int):
    _check(ctx, library().lbm_step(ctypes.c_void_p(ctx), int(n)))


def lbm_step_noalloc(ctx, n: int):
    _check(ctx, library().lbm_step_noalloc(ctypes.c_void_p(ctx), int(n)))


def lbm_read_macros(ctx, rho: int | None, u: int | None, T: int | None = None):
    _check(ctx, library().lbm_read_macros(ctypes.c_void_p(ctx), ctypes.c_void_p(rho or 0), ctypes.c_void_p(u or 0),
                                          ctypes.c_void_p(T or 0)))


def lbm_wall_force(ctx, n_groups: int = MAX_GROUPS) -> np.ndarray:
    out = np.zeros((n_groups, 4), np.float64)
    st = library().lbm_wall_force(ctypes.c_void_p(ctx), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                  int(n_groups))
    _check(ctx, st)
    return out


def lbm_diagnostics(ctx, n: int = LBM_DIAG_COUNT) -> np.ndarray:
    out = np.zeros(n, np.float64)
    st = library().lbm_diagnostics(ctypes.c_void_p(ctx), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(n))
    _check(ctx, st)
    return out


def lbm_time(ctx) -> int:
    return int(library().lbm_time(ctypes.c_void_p(ctx)))


def lbm_resume(ctx, t: int):
    _check(ctx, library().lbm_resume(ctypes.c_void_p(ctx), int(t)))


def lbm_num_links(ctx, lattice: int) -> int:
    return int(library().lbm_num_links(ctypes.c_void_p(ctx), int(lattice)))


def lbm_count_links(params: dict, labels, lattice: int) -> int:
    p = to_params(params)
    lp, _keep = _labels_ptr(labels, params)
    return int(library().lbm_count_links(ctypes.byref(p), lp, int(lattice)))


def lbm_check_links(params: dict, labels=None, dtype=4, streaming=LBM_STREAM_AUTO):
    """Raise LbmError if the links lbm_create would build store twice into
    one slot (host only)."""
    p = to_params(params, dtype, streaming)
    lp, _keep = _labels_ptr(labels, params)
    st = library().lbm_check_links(ctypes.byref(p), lp)
    if st != LBM_OK:
        raise LbmError(st, lbm_last_error(None))


def lbm_last_error(ctx) -> str:
    s = library().lbm_last_error(ctypes.c_void_p(ctx) if ctx else None)
    return s.decode() if s else ""


def lbm_destroy(ctx):
    if ctx:
        library().lbm_destroy(ctypes.c_void_p(ctx))


def lbm_profile(ctx, on: bool):
    _check(ctx, library().lbm_profile(ctypes.c_void_p(ctx), 1 if on else 0))


def lbm_profile_read(ctx, n: int = LBM_KERNEL_KINDS):
    """(milliseconds, launch counts) per kernel kind, numpy arrays of n."""
    ms = np.zeros(n, np.float64)
    launches = np.zeros(n, np.int64)
    st = library().lbm_profile_read(ctypes.c_void_p(ctx), ms.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                    launches.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(n))
    _check(ctx, st)
    return ms, launches


class Solver:
    """A context plus the torch-allocated device buffer it borrows.

    ``dtype`` is 4 (fp32) or 8 (fp64); ``streaming`` one of LBM_STREAM_*.
    Fields are passed and returned as torch tensors on the device (numpy
    inputs are copied to the device first); the stream is torch's current
    stream of the device unless one is given.
    """

    def __init__(self, params: dict, labels=None, dtype=4, streaming=LBM_STREAM_AUTO, device="cuda",
                 stream=None):
        import torch

        self.torch = torch
        self.params = dict(params)
        self.dtype = dtype
        self.tdtype = torch.float32 if dtype == 4 else torch.float64
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.cells = params["nx"] * params["ny"] * params["nz"]
        nbytes = lbm_required_bytes(params, labels, dtype, streaming)
        if nbytes == 0:
            raise LbmError(LBM_E_INVALID, "parameters rejected by lbm_required_bytes")
        self.nbytes = nbytes
        # allocated on the solver's stream, where every use of it is queued, so
        # that torch reuses the memory only after that work
        with torch.cuda.stream(self.stream):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.ctx = lbm_create(params, labels, self.buf.data_ptr(), nbytes, self.stream.cuda_stream, dtype, streaming)
        self._keep = None

    def _dev(self, a, shape):
        t = self.torch
        if a is None:
            return None
        if not isinstance(a, t.Tensor):
            a = t.from_numpy(np.ascontiguousarray(a))
        return a.to(device=self.device, dtype=self.tdtype).reshape(shape).contiguous()

    def init(self, rho, u, T=None):
        n = self.cells
        # the inputs may come from work on the caller's stream: the solver's
        # stream waits for it, then converts, copies and reads them itself
        self.stream.wait_stream(self.torch.cuda.current_stream(self.device))
        with self.torch.cuda.stream(self.stream):
            rho_d, u_d, T_d = self._dev(rho, (n,)), self._dev(u, (3, n)), self._dev(T, (n,))
            lbm_init_fields(self.ctx, rho_d.data_ptr(), u_d.data_ptr(), T_d.data_ptr() if T_d is not None else 0)
        self._keep = (rho, u, T, rho_d, u_d, T_d)  # read by a copy or a kernel on the stream

    def step(self, n: int):
        lbm_step(self.ctx, n)

    def step_noalloc(self, n: int):
        """The same steps through lbm_step_noalloc (no allocation, no replay
        graph; scratch in the library's static per-GPU array)."""
        lbm_step_noalloc(self.ctx, n)

    def macros(self):
        """(rho, u[3, n], T or None) as device tensors, written on the
        solver's stream; the caller's current stream waits for them."""
        t = self.torch
        n = self.cells
        caller = t.cuda.current_stream(self.device)
        with t.cuda.stream(self.stream):
            rho = t.empty(n, dtype=self.tdtype, device=self.device)
            u = t.empty((3, n), dtype=self.tdtype, device=self.device)
            T = t.empty(n, dtype=self.tdtype, device=self.device) if self.params.get("thermal") else None
            lbm_read_macros(self.ctx, rho.data_ptr(), u.data_ptr(), T.data_ptr() if T is not None else 0)
        caller.wait_stream(self.stream)
        for x in (rho, u, T):
            if x is not None and caller != self.stream:
                x.record_stream(caller)
        return rho, u, T

    def wall_force(self, n_groups: int = MAX_GROUPS) -> np.ndarray:
        return lbm_wall_force(self.ctx, n_groups)

    def diagnostics(self) -> np.ndarray:
        return lbm_diagnostics(self.ctx)

    @property
    def time(self) -> int:
        return lbm_time(self.ctx)

    def num_links(self, lattice: int) -> int:
        return lbm_num_links(self.ctx, lattice)

    def profile(self, on: bool = True):
        """Switch per-kernel timing on (sums restart at zero) or off."""
        lbm_profile(self.ctx, on)

    def kernel_times(self) -> dict:
        """{kernel kind: (milliseconds, launches)} for the kinds launched since
        profiling was switched on."""
        ms, launches = lbm_profile_read(self.ctx)
        return {KERNEL_NAMES[k]: (float(ms[k]), int(launches[k])) for k in range(LBM_KERNEL_KINDS) if launches[k]}

    def checkpoint(self):
        """A checkpoint: a copy of the buffer's bytes (device tensor), taken on
        the solver's stream after the work queued so far, and the time."""
        with self.torch.cuda.stream(self.stream):
            saved = self.buf.clone()
        self.stream.synchronize()
        return saved, self.time

    def resume(self, saved, t: int):
        """Continue from a checkpoint of a solver with the same parameters,
        labels, dtype and streaming mode (in place of init)."""
        if saved.numel() != self.buf.numel():
            raise LbmError(LBM_E_INVALID, "checkpoint size differs from this solver's buffer")
        with self.torch.cuda.stream(self.stream):
            self.buf.copy_(saved, non_blocking=True)
            self._keep = saved  # read by the copy on the stream
        lbm_resume(self.ctx, t)

    def close(self):
        if self.ctx:
            lbm_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
