"""ctypes wrapper of ``lbm_oracle.c`` (test infrastructure; see package docstring).

Every function takes a plain parameter dict (the one the seeded input
generators produce) and numpy arrays, and returns numpy arrays.  Field arrays
use the index ``x + nx*(y + ny*z)``; vector fields are three such planes;
populations are ``[q][cell]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lbm_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

Q19 = 19
Q7 = 7
Q9 = 9
Q5 = 5
MAX_GROUPS = 261  # 6 faces + 255 solid labels


class OracleParams(ctypes.Structure):
    """Mirror of ``oracle_params`` in lbm_oracle.c (the oracle's own struct)."""

    _fields_ = [
        ("nx", ctypes.c_int32),
        ("ny", ctypes.c_int32),
        ("nz", ctypes.c_int32),
        ("thermal", ctypes.c_int32),
        ("face_kind", ctypes.c_int32 * 6),
        ("face_thermal", ctypes.c_int32 * 6),
        ("face_T", ctypes.c_double * 6),
        ("solid_thermal", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
        ("solid_T", ctypes.c_double),
        ("s19", ctypes.c_double * 19),
        ("s7", ctypes.c_double * 7),
        ("a_T", ctypes.c_double),
        ("accel", ctypes.c_double * 3),
        ("gbeta", ctypes.c_double * 3),
        ("T0", ctypes.c_double),
        ("face_u", ctypes.c_double * 18),
        ("face_rho", ctypes.c_double * 6),
        ("lattice", ctypes.c_int32),
        ("pad1", ctypes.c_int32),
        ("s9", ctypes.c_double * 9),
        ("s5", ctypes.c_double * 5),
    ]


def library_path() -> str:
    return _SO


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_tables.argtypes = [ip, dp, ip, dp, dp, ip, ip, dp, dp]
        lib.oracle_tables.restype = ctypes.c_int
        lib.oracle_tables_2d.argtypes = [ip, dp, ip, dp, dp, ip, ip, dp, dp]
        lib.oracle_tables_2d.restype = ctypes.c_int
        lib.oracle_collide.argtypes = [ctypes.POINTER(OracleParams), ctypes.c_int64, dp, dp, dp, dp, dp]
        lib.oracle_collide.restype = ctypes.c_int
        lib.oracle_equilibrium.argtypes = [ctypes.POINTER(OracleParams), ctypes.c_int64, dp, dp, dp, dp, dp]
        lib.oracle_equilibrium.restype = ctypes.c_int
        lib.oracle_run.argtypes = [
            ctypes.POINTER(OracleParams), ctypes.POINTER(ctypes.c_uint8), ip, ip,
            dp, dp, dp, dp, dp, ctypes.c_int32, dp, dp, dp, dp, dp, dp, ctypes.c_int32, ctypes.c_int32,
        ]
        lib.oracle_run.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def _dp(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def to_params(d: dict) -> OracleParams:
    """Marshal the shared parameter dict into the oracle's struct."""
    p = OracleParams()
    p.nx, p.ny, p.nz = int(d["nx"]), int(d["ny"]), int(d["nz"])
    p.thermal = int(d.get("thermal", 0))
    for i in range(6):
        p.face_kind[i] = int(d.get("face_kind", [0] * 6)[i])
        p.face_thermal[i] = int(d.get("face_thermal", [0] * 6)[i])
        p.face_T[i] = float(d.get("face_T", [0.0] * 6)[i])
    p.solid_thermal = int(d.get("solid_thermal", 0))
    p.solid_T = float(d.get("solid_T", 0.0))
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
    p.lattice = int(d.get("lattice", 0))
    if p.lattice == 0:
        for i in range(19):
            p.s19[i] = float(d["s19"][i])
        for i in range(7):
            p.s7[i] = float(d.get("s7", [0.0] * 7)[i])
    else:
        for i in range(9):
            p.s9[i] = float(d["s9"][i])
        for i in range(5):
            p.s5[i] = float(d.get("s5", [0.0] * 5)[i])
    return p


def lattice_sizes(params: dict) -> tuple:
    """(Q, QT): velocities of the flow and temperature lattices in use."""
    return (Q9, Q5) if int(params.get("lattice", 0)) == 1 else (Q19, Q7)


def tables() -> dict:
    """Velocity sets, weights, opposites and moment matrices as the oracle built them."""
    lib = _lib()
    c19 = np.zeros((Q19, 3), np.int32)
    w19 = np.zeros(Q19)
    opp19 = np.zeros(Q19, np.int32)
    m19 = np.zeros((Q19, Q19))
    minv19 = np.zeros((Q19, Q19))
    c7 = np.zeros((Q7, 3), np.int32)
    opp7 = np.zeros(Q7, np.int32)
    n7 = np.zeros((Q7, Q7))
    ninv7 = np.zeros((Q7, Q7))
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = lib.oracle_tables(c19.ctypes.data_as(ip), _dp(w19), opp19.ctypes.data_as(ip), _dp(m19),
                           _dp(minv19), c7.ctypes.data_as(ip), opp7.ctypes.data_as(ip), _dp(n7), _dp(ninv7))
    if rc:
        raise RuntimeError("oracle_tables failed")
    return dict(c19=c19, w19=w19, opp19=opp19, M=m19, Minv=minv19, c7=c7, opp7=opp7, N=n7, Ninv=ninv7)


def tables_2d() -> dict:
    """The two-dimensional pair (D2Q9, D2Q5) as the oracle built it."""
    lib = _lib()
    c9 = np.zeros((Q9, 3), np.int32)
    w9 = np.zeros(Q9)
    opp9 = np.zeros(Q9, np.int32)
    m9 = np.zeros((Q9, Q9))
    minv9 = np.zeros((Q9, Q9))
    c5 = np.zeros((Q5, 3), np.int32)
    opp5 = np.zeros(Q5, np.int32)
    n5 = np.zeros((Q5, Q5))
    ninv5 = np.zeros((Q5, Q5))
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = lib.oracle_tables_2d(c9.ctypes.data_as(ip), _dp(w9), opp9.ctypes.data_as(ip), _dp(m9),
                              _dp(minv9), c5.ctypes.data_as(ip), opp5.ctypes.data_as(ip), _dp(n5), _dp(ninv5))
    if rc:
        raise RuntimeError("oracle_tables_2d failed")
    return dict(c9=c9, w9=w9, opp9=opp9, M=m9, Minv=minv9, c5=c5, opp5=opp5, N=n5, Ninv=ninv5)


def collide(params: dict, f, g=None):
    """Collide cells given cell-major: f[n,Q], g[n,QT] (19 and 7, or 9 and 5).

    Returns (fpost, gpost, mac[n,5])."""
    p = to_params(params)
    f = _f64(np.atleast_2d(f))
    n = f.shape[0]
    fpost = np.zeros_like(f)
    mac = np.zeros((n, 5))
    gpost = None
    if p.thermal:
        g = _f64(np.atleast_2d(g))
        gpost = np.zeros_like(g)
    rc = _lib().oracle_collide(ctypes.byref(p), n, _dp(f), _dp(g), _dp(fpost), _dp(gpost), _dp(mac))
    if rc:
        raise RuntimeError("oracle_collide failed")
    return fpost, gpost, mac


def equilibrium(params: dict, rho, u, T=None):
    """f_eq[n,Q] (and g_eq[n,QT]) for cell-major rho[n], u[n,3], T[n]."""
    p = to_params(params)
    Q, QT = lattice_sizes(params)
    rho = _f64(np.atleast_1d(rho))
    u = _f64(np.atleast_2d(u))
    n = rho.shape[0]
    feq = np.zeros((n, Q))
    geq = np.zeros((n, QT)) if T is not None else None
    T = _f64(np.atleast_1d(T)) if T is not None else None
    rc = _lib().oracle_equilibrium(ctypes.byref(p), n, _dp(rho), _dp(u), _dp(T), _dp(feq), _dp(geq))
    if rc:
        raise RuntimeError("oracle_equilibrium failed")
    return feq, geq


def run(params: dict, nsteps: int, rho0=None, u0=None, T0=None, labels=None, window=None,
        f0=None, g0=None, want_populations=False, want_diag=False, ngroups=MAX_GROUPS,
        nthreads=0):
    """Run ``nsteps`` collide-then-stream steps.

    window: ((lo_x, lo_y, lo_z), (n_x, n_y, n_z)) or None for the whole box.
    rho0/u0/T0 are window-local fields (u0 shaped [3, cells]); labels is the
    full box (uint8, 0 = fluid).  Returns a dict with rho, u[3,cells], T and
    optionally f[Q,cells], g[QT,cells], diag[nsteps, ngroups, 4].
    """
    p = to_params(params)
    Q, QT = lattice_sizes(params)
    N = (p.nx, p.ny, p.nz)
    if window is None:
        lo, wn = (0, 0, 0), N
    else:
        lo, wn = window
    cells = int(wn[0]) * int(wn[1]) * int(wn[2])
    lo_a = (ctypes.c_int32 * 3)(*[int(v) for v in lo])
    wn_a = (ctypes.c_int32 * 3)(*[int(v) for v in wn])
    lab_ptr = ctypes.POINTER(ctypes.c_uint8)()
    if labels is not None:
        labels = np.ascontiguousarray(labels, dtype=np.uint8).reshape(-1)
        assert labels.size == N[0] * N[1] * N[2]
        lab_ptr = labels.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    rho0 = _f64(rho0)
    u0 = _f64(u0)
    T0 = _f64(T0)
    f0 = _f64(f0)
    g0 = _f64(g0)
    if f0 is None:
        assert rho0 is not None and rho0.size == cells and u0.size == 3 * cells
        if p.thermal:
            assert T0 is not None and T0.size == cells
    else:
        assert f0.size == Q * cells
        if p.thermal:
            assert g0 is not None and g0.size == QT * cells
    rho = np.zeros(cells)
    u = np.zeros((3, cells))
    T = np.zeros(cells)
    fo = np.zeros((Q, cells)) if want_populations else None
    go = np.zeros((QT, cells)) if (want_populations and p.thermal) else None
    diag = np.zeros((max(nsteps, 0), ngroups, 4)) if want_diag else None
    rc = _lib().oracle_run(ctypes.byref(p), lab_ptr, lo_a, wn_a, _dp(rho0), _dp(u0), _dp(T0), _dp(f0),
                           _dp(g0), int(nsteps), _dp(rho), _dp(u), _dp(T), _dp(fo), _dp(go), _dp(diag),
                           int(ngroups), int(nthreads))
    if rc:
        raise RuntimeError("oracle_run rejected its arguments")
    out = dict(rho=rho, u=u, T=T)
    if want_populations:
        out["f"] = fo
        out["g"] = go
    if want_diag:
        out["diag"] = diag
    return out
