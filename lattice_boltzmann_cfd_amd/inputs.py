"""Seeded synthetic inputs: parameter recipes, initial fields, solid labels.

This module holds none of the method's per-step arithmetic.  It only makes the
inputs that both the HIP library (through its binding) and the CPU oracle
consume: a plain parameter dict, the initial density / velocity / temperature
fields and the uint8 solid-label array.

Field arrays are numpy fp64 with the flat cell index ``x + nx*(y + ny*z)``;
velocity is three such planes, ``u[3, cells]``.

Workloads (the pages give no input data; every one is synthetic):
  * ``tg32``     -- D3Q19 MRT, 32^3 periodic, Taylor-Green vortex u0=0.05 plus
                    seeded uniform +-1e-3 density noise, tau = 0.6.
  * ``sol128``   -- 128^3 periodic, tau = 0.55, random solenoidal field
                    (curl of a random vector potential, modes 1 <= |k| <= 4),
                    scaled to max|u| = 0.05 on rho = 1.
  * ``sphere128``-- 128^3 periodic, centred solid sphere R = 16, body force
                    gx = 1e-6, tau = 0.6, fluid at rest.
  * ``cavity256``-- thermal D3Q19 + D3Q7, 256^3 closed cavity, x- hot (+0.5),
                    x+ cold (-0.5), other faces adiabatic, Pr = 0.71,
                    Ra = 1e7, buoyancy along +z.
  * ``rb512``    -- thermal, 512^3, periodic in x/y, z- hot (+0.5), z+ cold
                    (-0.5), seeded random non-overlapping spheres of radius
                    4..12 up to 10 % solid fraction, Ra = 1e8, Pr = 0.71.
  * ``sol256``   -- the ``sol128`` recipe at 256^3 (the throughput point).
  * ``sol512``   -- the same recipe at 512^3 (the largest isothermal box).
  * ``channel256``-- flow past a sphere in an open channel, 256x128x128: x-
                    a velocity inlet at U = 0.05, x+ a pressure outlet at
                    rho_w = 1, y and z free-slip faces, a solid sphere R = 16
                    at (nx/4, ny/2, nz/2), tau = 0.52, uniform start u = (U,
                    0, 0) on rho = 1 (exercises the slip, velocity and
                    pressure face rules).
  * ``cavity2d`` -- thermal D2Q9 + D2Q5 (the thermal-LBM page's 2D model),
                    8193 x 8193 square cell, x- hot (+0.5), x+ cold (-0.5),
                    y faces adiabatic, no-slip everywhere, Pr = 0.71,
                    Ra = 1e8, buoyancy along +y, fp64 (the page runs its 2D
                    cell in double precision for 12000 steps).
  * ``tg2d``     -- D2Q9 MRT, 256 x 256 periodic Taylor-Green vortex u0 =
                    0.05 with +-1e-3 density noise, tau = 0.6.

Relaxation-rate slots follow the moment basis row order used by both sides:
0 rho, 1 e, 2 eps, 3/5/7 j, 4/6/8 q, 9 3pxx, 10 3pixx, 11 pww, 12 piww,
13-15 pxy/pyz/pxz, 16-18 m.  D3Q7 rows: 0 T, 1-3 flux, 4 energy-like,
5-6 second-order anisotropic.  Two-dimensional runs (``lattice = 1``, nz = 1)
use ``s9`` in the D2Q9 row order 0 rho, 1 e, 2 eps, 3 jx, 4 qx, 5 jy, 6 qy,
7 pxx, 8 pxy and ``s5`` in the D2Q5 row order 0 T, 1-2 flux, 3 energy-like,
4 anisotropic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

FACE_PERIODIC = 0
FACE_WALL = 1
FACE_SLIP = 2
FACE_VELOCITY = 3
FACE_PRESSURE = 4
ADIABATIC = 0
DIRICHLET = 1

ROWS_NU = (9, 11, 13, 14, 15)
ROWS_Q = (4, 6, 8)
ROWS_PI = (10, 12)
ROWS_M = (16, 17, 18)

# default free-fall velocity in lattice units for the thermal workloads
U_FREEFALL = 0.1
# default D3Q7 constant a_T (rest weight (1 - a_T)/7 = 1/4)
A_T_DEFAULT = -0.75
# default D2Q5 constant a_T: rest weight (1 - a_T)/5 = 1/2, moving (4 + a_T)/20
# = 1/8, the weights the D3Q7 default sums to on a single z layer
A_T_DEFAULT_2D = -1.5
ROWS_NU_2D = (7, 8)
ROWS_Q_2D = (4, 6)


def mrt_rates(tau: float, s_e=1.19, s_eps=1.4, s_q=1.2, s_pi=1.4, s_m=1.98) -> list:
    """D3Q19 rates: s_nu = 1/tau on the five stress rows, conserved rows 0."""
    s = [0.0] * 19
    s[1] = s_e
    s[2] = s_eps
    for r in ROWS_Q:
        s[r] = s_q
    for r in ROWS_NU:
        s[r] = 1.0 / tau
    for r in ROWS_PI:
        s[r] = s_pi
    for r in ROWS_M:
        s[r] = s_m
    return s


def poiseuille_rates(tau: float) -> list:
    """Rates with s_q = s_m = 8(2 - s_nu)/(8 - s_nu) (wall exactly half-way)."""
    s_nu = 1.0 / tau
    magic = 8.0 * (2.0 - s_nu) / (8.0 - s_nu)
    return mrt_rates(tau, s_q=magic, s_m=magic)


def bgk_rates(tau: float) -> list:
    """Every row relaxed at 1/tau (the MRT operator then reduces to BGK)."""
    return [1.0 / tau] * 19


def thermal_rates(alpha: float, a_T: float = A_T_DEFAULT, q_e: float = 1.0, q_nu: float = 1.0) -> list:
    """D3Q7 rates: q_kappa on the flux rows from alpha = cs_T^2 (1/q_kappa - 1/2)."""
    cs2 = (6.0 + a_T) / 21.0
    q_k = 1.0 / (alpha / cs2 + 0.5)
    return [0.0, q_k, q_k, q_k, q_e, q_nu, q_nu]


def mrt_rates_2d(tau: float, s_e=1.1, s_eps=1.0, s_q=1.2) -> list:
    """D2Q9 rates: s_nu = 1/tau on the two stress rows, conserved rows 0."""
    s = [0.0] * 9
    s[1] = s_e
    s[2] = s_eps
    for r in ROWS_Q_2D:
        s[r] = s_q
    for r in ROWS_NU_2D:
        s[r] = 1.0 / tau
    return s


def poiseuille_rates_2d(tau: float) -> list:
    """D2Q9 rates with s_q = 8(2 - s_nu)/(8 - s_nu) (wall exactly half-way)."""
    s_nu = 1.0 / tau
    return mrt_rates_2d(tau, s_q=8.0 * (2.0 - s_nu) / (8.0 - s_nu))


def thermal_rates_2d(alpha: float, a_T: float = A_T_DEFAULT_2D, q_e: float = 1.0, q_nu: float = 1.0) -> list:
    """D2Q5 rates: q_kappa on the flux rows from alpha = cs_T^2 (1/q_kappa - 1/2),
    cs_T^2 = (4 + a_T)/10."""
    cs2 = (4.0 + a_T) / 10.0
    q_k = 1.0 / (alpha / cs2 + 0.5)
    return [0.0, q_k, q_k, q_e, q_nu]


def thermal_scales(H: float, Ra: float, Pr: float, U_f: float = U_FREEFALL) -> dict:
    """Lattice parameters from Ra = g beta dT H^3/(nu alpha), Pr = nu/alpha, dT = 1,
    free-fall velocity U_f = sqrt(g beta dT H)."""
    gbeta = U_f * U_f / H
    nu = U_f * H * math.sqrt(Pr / Ra)
    alpha = nu / Pr
    return dict(gbeta=gbeta, nu=nu, alpha=alpha, tau=3.0 * nu + 0.5)


def base_params(nx, ny, nz, s19, thermal=False, face_kind=None, face_thermal=None, face_T=None,
                s7=None, a_T=A_T_DEFAULT, accel=(0.0, 0.0, 0.0), gbeta=(0.0, 0.0, 0.0), T0=0.0,
                solid_thermal=ADIABATIC, solid_T=0.0, face_u=None, face_rho=None) -> dict:
    """face_u: 6 wall velocities (3 components each) of VELOCITY faces;
    face_rho: 6 wall densities of VELOCITY and PRESSURE faces."""
    fu = [0.0] * 18 if face_u is None else [float(v) for v in np.asarray(face_u, dtype=float).reshape(-1)]
    return dict(
        nx=int(nx), ny=int(ny), nz=int(nz), thermal=int(bool(thermal)),
        face_kind=list(face_kind or [FACE_PERIODIC] * 6),
        face_thermal=list(face_thermal or [ADIABATIC] * 6),
        face_T=list(face_T or [0.0] * 6),
        s19=list(s19), s7=list(s7 or [0.0] * 7), a_T=float(a_T),
        accel=list(accel), gbeta=list(gbeta), T0=float(T0),
        solid_thermal=int(solid_thermal), solid_T=float(solid_T),
        face_u=fu, face_rho=list(face_rho or [1.0] * 6),
    )


def base_params_2d(nx, ny, s9, thermal=False, face_kind=None, face_thermal=None, face_T=None, s5=None,
                   a_T=A_T_DEFAULT_2D, accel=(0.0, 0.0), gbeta=(0.0, 0.0), T0=0.0, solid_thermal=ADIABATIC,
                   solid_T=0.0, face_u=None, face_rho=None) -> dict:
    """Parameters of a two-dimensional run (D2Q9 + D2Q5, lattice = 1) on one
    periodic z layer.  face_kind, face_thermal, face_T, face_rho: 4 values
    (x-, x+, y-, y+); face_u: 4 wall velocities (ux, uy); accel, gbeta: 2
    components."""
    def six(v, fill):
        v = list(v) if v is not None else [fill] * 4
        return v[:4] + [fill, fill]
    fu = np.zeros((6, 3))
    if face_u is not None:
        fu[:4, :2] = np.asarray(face_u, dtype=float).reshape(4, 2)
    d = base_params(nx, ny, 1, [0.0] * 19, thermal=thermal, face_kind=six(face_kind, FACE_PERIODIC),
                    face_thermal=six(face_thermal, ADIABATIC), face_T=six(face_T, 0.0), a_T=a_T,
                    accel=(accel[0], accel[1], 0.0), gbeta=(gbeta[0], gbeta[1], 0.0), T0=T0,
                    solid_thermal=solid_thermal, solid_T=solid_T, face_u=fu, face_rho=six(face_rho, 1.0))
    d["lattice"] = 1
    d["s9"] = [float(v) for v in s9]
    d["s5"] = [float(v) for v in (s5 or [0.0] * 5)]
    return d


# ------------------------------------------------------------------ fields

def cell_coords(nx, ny, nz):
    z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    return x.reshape(-1).astype(np.float64), y.reshape(-1).astype(np.float64), z.reshape(-1).astype(np.float64)


def taylor_green(nx, ny, nz, u0=0.05, noise=1e-3, seed=1):
    """u = u0 (sin kx cos ky cos kz, -cos kx sin ky cos kz, 0), k = 2 pi / n per axis
    (on node coordinates x = i), rho = 1 + U(-noise, noise)."""
    x, y, z = cell_coords(nx, ny, nz)
    kx, ky, kz = 2 * math.pi / nx, 2 * math.pi / ny, 2 * math.pi / nz
    u = np.zeros((3, nx * ny * nz))
    u[0] = u0 * np.sin(kx * x) * np.cos(ky * y) * np.cos(kz * z)
    u[1] = -u0 * np.cos(kx * x) * np.sin(ky * y) * np.cos(kz * z)
    rng = np.random.default_rng(seed)
    rho = 1.0 + rng.uniform(-noise, noise, size=nx * ny * nz)
    return rho, u


def solenoidal(nx, ny, nz, umax=0.05, kmax=4, seed=2):
    """Real part of the spectral curl of a random vector potential with N(0,1)
    complex coefficients on integer wavevectors 1 <= |k| <= kmax, scaled so that
    max |u| = umax.  Divergence-free in the continuum."""
    rng = np.random.default_rng(seed)
    uh = np.zeros((3, nz, ny, nx), np.complex128)
    for kz in range(-kmax, kmax + 1):
        for ky in range(-kmax, kmax + 1):
            for kx in range(-kmax, kmax + 1):
                k2 = kx * kx + ky * ky + kz * kz
                if k2 < 1 or k2 > kmax * kmax:
                    continue
                a = rng.standard_normal(3) + 1j * rng.standard_normal(3)
                k = np.array([kx, ky, kz], np.float64)
                c = 1j * np.cross(k, a)  # curl in Fourier space
                uh[:, kz % nz, ky % ny, kx % nx] += c
    u = np.real(np.fft.ifftn(uh, axes=(1, 2, 3))) * (nx * ny * nz)
    u = u.reshape(3, -1)
    scale = umax / np.sqrt((u * u).sum(axis=0)).max()
    u *= scale
    rho = np.ones(nx * ny * nz)
    return rho, u


def rest(nx, ny, nz):
    n = nx * ny * nz
    return np.ones(n), np.zeros((3, n)), np.zeros(n)


# ------------------------------------------------------------------ solids

def sphere_labels(nx, ny, nz, R, centre=None, label=1):
    """A cell is solid iff |(i+1/2, j+1/2, k+1/2) - centre| <= R."""
    if centre is None:
        centre = (nx / 2.0, ny / 2.0, nz / 2.0)
    x, y, z = cell_coords(nx, ny, nz)
    d2 = (x + 0.5 - centre[0]) ** 2 + (y + 0.5 - centre[1]) ** 2 + (z + 0.5 - centre[2]) ** 2
    lab = np.zeros(nx * ny * nz, np.uint8)
    lab[d2 <= R * R] = label
    return lab


def random_spheres(nx, ny, nz, rmin=4, rmax=12, fraction=0.10, seed=5, label=1, max_tries=2_000_000):
    """Non-overlapping spheres, integer radius U[rmin, rmax], centre uniform in
    x, y and in z in [R, nz - R]; a candidate is kept when its distance to every
    kept sphere (minimum image in the periodic x, y) exceeds R1 + R2.  Spheres are
    added until the voxel solid fraction reaches ``fraction``."""
    rng = np.random.default_rng(seed)
    lab = np.zeros((nz, ny, nx), np.uint8)
    cs = np.zeros((0, 3))
    rs = np.zeros(0)
    target = fraction * nx * ny * nz
    solid = 0
    tries = 0
    spheres = []
    while solid < target:
        tries += 1
        if tries > max_tries:
            raise RuntimeError("random_spheres: could not reach the solid fraction")
        R = int(rng.integers(rmin, rmax + 1))
        c = np.array([rng.uniform(0, nx), rng.uniform(0, ny), rng.uniform(R, nz - R)])
        if len(rs):
            d = cs - c
            d[:, 0] -= nx * np.round(d[:, 0] / nx)
            d[:, 1] -= ny * np.round(d[:, 1] / ny)
            if np.any(np.sqrt((d * d).sum(axis=1)) <= rs + R):
                continue
        cs = np.vstack([cs, c])
        rs = np.append(rs, R)
        spheres.append((float(c[0]), float(c[1]), float(c[2]), R))
        # voxelise within the bounding box, wrapping x and y
        zr = np.arange(max(0, int(math.floor(c[2] - R - 1))), min(nz, int(math.ceil(c[2] + R + 1)) + 1))
        yr = np.arange(int(math.floor(c[1] - R - 1)), int(math.ceil(c[1] + R + 1)) + 1)
        xr = np.arange(int(math.floor(c[0] - R - 1)), int(math.ceil(c[0] + R + 1)) + 1)
        Z, Y, X = np.meshgrid(zr, yr, xr, indexing="ij")
        d2 = (X + 0.5 - c[0]) ** 2 + (Y + 0.5 - c[1]) ** 2 + (Z + 0.5 - c[2]) ** 2
        inside = d2 <= R * R
        zi, yi, xi = Z[inside], Y[inside] % ny, X[inside] % nx
        before = int(np.count_nonzero(lab[zi, yi, xi]))
        lab[zi, yi, xi] = label
        solid += int(inside.sum()) - before
    return lab.reshape(-1), spheres


# --------------------------------------------------------------- workloads

@dataclass
class Workload:
    name: str
    params: dict
    rho: np.ndarray
    u: np.ndarray
    T: np.ndarray | None
    labels: np.ndarray | None
    steps: int
    info: dict = field(default_factory=dict)

    @property
    def shape(self):
        return (self.params["nx"], self.params["ny"], self.params["nz"])

    @property
    def cells(self):
        return self.params["nx"] * self.params["ny"] * self.params["nz"]


def tg32(shape=(32, 32, 32), seed=1) -> Workload:
    nx, ny, nz = shape
    rho, u = taylor_green(nx, ny, nz, seed=seed)
    p = base_params(nx, ny, nz, mrt_rates(0.6))
    return Workload("tg32", p, rho, u, None, None, 100)


def sol128(shape=(128, 128, 128), seed=2, tau=0.55) -> Workload:
    nx, ny, nz = shape
    rho, u = solenoidal(nx, ny, nz, seed=seed)
    p = base_params(nx, ny, nz, mrt_rates(tau))
    return Workload("sol128", p, rho, u, None, None, 1000)


def sol256(shape=(256, 256, 256), seed=2) -> Workload:
    w = sol128(shape, seed=seed)
    w.name = "sol256"
    return w


def sol512(shape=(512, 512, 512), seed=2) -> Workload:
    w = sol128(shape, seed=seed)
    w.name = "sol512"
    return w


def sphere128(shape=(128, 128, 128), R=16.0, gx=1e-6, tau=0.6) -> Workload:
    nx, ny, nz = shape
    rho, u, _ = rest(nx, ny, nz)
    lab = sphere_labels(nx, ny, nz, R)
    p = base_params(nx, ny, nz, mrt_rates(tau), accel=(gx, 0.0, 0.0))
    return Workload("sphere128", p, rho, u, None, lab, 2000, dict(R=R))


def cavity256(shape=(256, 256, 256), Ra=1e7, Pr=0.71, H=256) -> Workload:
    nx, ny, nz = shape
    sc = thermal_scales(H, Ra, Pr)
    rho, u, T = rest(nx, ny, nz)
    p = base_params(
        nx, ny, nz, mrt_rates(sc["tau"]), thermal=True,
        face_kind=[FACE_WALL] * 6,
        face_thermal=[DIRICHLET, DIRICHLET, ADIABATIC, ADIABATIC, ADIABATIC, ADIABATIC],
        face_T=[0.5, -0.5, 0.0, 0.0, 0.0, 0.0],
        s7=thermal_rates(sc["alpha"]), gbeta=(0.0, 0.0, sc["gbeta"]), T0=0.0,
    )
    return Workload("cavity256", p, rho, u, T, None, 5000, dict(scales=sc, Ra=Ra, Pr=Pr, H=H))


def cavity385(shape=(385, 385, 385), Ra=1e7, Pr=0.71, H=None) -> Workload:
    """The thermal-LBM page's 3D strong-scaling grid (Sec. 2: 385^3, odd so
    that the half-way walls put a cell on the centre plane; 6000 steps, run
    in double precision there) with the heated-cavity recipe of cavity256 (the
    page's Rayleigh number for it is not printed); H defaults to the box
    width."""
    H = shape[0] if H is None else H
    w = cavity256(shape, Ra=Ra, Pr=Pr, H=H)
    return Workload("cavity385", w.params, w.rho, w.u, w.T, None, 6000, w.info)


def rb512(shape=(512, 512, 512), Ra=1e8, Pr=0.71, H=512, seed=5, rmin=4, rmax=12) -> Workload:
    """Reduced boxes keep the recipe; the largest radius is clamped to
    (nz - 1)//2 - 1 so that a sphere fits between the plates."""
    nx, ny, nz = shape
    sc = thermal_scales(H, Ra, Pr)
    rho, u, T = rest(nx, ny, nz)
    rmax = max(rmin, min(rmax, (nz - 1) // 2 - 1))
    lab, spheres = random_spheres(nx, ny, nz, rmin=rmin, rmax=rmax, seed=seed)
    p = base_params(
        nx, ny, nz, mrt_rates(sc["tau"]), thermal=True,
        face_kind=[FACE_PERIODIC, FACE_PERIODIC, FACE_PERIODIC, FACE_PERIODIC, FACE_WALL, FACE_WALL],
        face_thermal=[ADIABATIC, ADIABATIC, ADIABATIC, ADIABATIC, DIRICHLET, DIRICHLET],
        face_T=[0.0, 0.0, 0.0, 0.0, 0.5, -0.5],
        s7=thermal_rates(sc["alpha"]), gbeta=(0.0, 0.0, sc["gbeta"]), T0=0.0,
        solid_thermal=ADIABATIC,
    )
    return Workload("rb512", p, rho, u, T, lab, 1000, dict(scales=sc, Ra=Ra, Pr=Pr, H=H, spheres=len(spheres)))


def channel256(shape=(256, 128, 128), U=0.05, R=16.0, tau=0.52, thermal=False) -> Workload:
    """Reduced boxes keep the recipe (sphere at a quarter of the length, on
    the axis).  With thermal=True the inflow carries T = 0.5 into a T = 0
    channel (Dirichlet inlet, adiabatic elsewhere) and the sphere is held at
    T = -0.5."""
    nx, ny, nz = shape
    rho = np.ones(nx * ny * nz)
    u = np.zeros((3, rho.size))
    u[0] = U
    lab = sphere_labels(nx, ny, nz, R, centre=(nx / 4.0, ny / 2.0, nz / 2.0))
    fu = np.zeros((6, 3))
    fu[0] = (U, 0.0, 0.0)
    kw = {}
    T = None
    if thermal:
        T = np.zeros(rho.size)
        kw = dict(thermal=True, s7=thermal_rates(0.02), face_thermal=[DIRICHLET, 0, 0, 0, 0, 0],
                  face_T=[0.5, 0, 0, 0, 0, 0], solid_thermal=DIRICHLET, solid_T=-0.5, gbeta=(0.0, 0.0, 1e-4))
    p = base_params(nx, ny, nz, mrt_rates(tau),
                    face_kind=[FACE_VELOCITY, FACE_PRESSURE, FACE_SLIP, FACE_SLIP, FACE_SLIP, FACE_SLIP],
                    face_u=fu, face_rho=[1.0] * 6, **kw)
    return Workload("channel256", p, rho, u, T, lab, 2000, dict(U=U, R=R))


def cavity2d(shape=(8193, 8193), Ra=1e8, Pr=0.71, H=None) -> Workload:
    """The thermal-LBM page's 2D convection cell (Sec. 2, Sec. 3 strong
    scaling grid 8193 x 8193).  Reduced boxes keep the recipe; H defaults to
    the box width."""
    nx, ny = shape[0], shape[1]
    H = nx if H is None else H
    sc = thermal_scales(H, Ra, Pr)
    rho, u, T = rest(nx, ny, 1)
    p = base_params_2d(
        nx, ny, mrt_rates_2d(sc["tau"]), thermal=True, face_kind=[FACE_WALL] * 4,
        face_thermal=[DIRICHLET, DIRICHLET, ADIABATIC, ADIABATIC], face_T=[0.5, -0.5, 0.0, 0.0],
        s5=thermal_rates_2d(sc["alpha"]), gbeta=(0.0, sc["gbeta"]), T0=0.0,
    )
    return Workload("cavity2d", p, rho, u, T, None, 12000, dict(scales=sc, Ra=Ra, Pr=Pr, H=H))


def tg2d(shape=(256, 256), u0=0.05, seed=1, tau=0.6) -> Workload:
    nx, ny = shape[0], shape[1]
    rho, u = taylor_green(nx, ny, 1, u0=u0, seed=seed)
    u[2] = 0.0
    p = base_params_2d(nx, ny, mrt_rates_2d(tau))
    return Workload("tg2d", p, rho, u, None, None, 1000)


WORKLOADS = dict(tg32=tg32, sol128=sol128, sol256=sol256, sol512=sol512, sphere128=sphere128, cavity256=cavity256,
                 cavity385=cavity385, rb512=rb512,
                 channel256=channel256, cavity2d=cavity2d, tg2d=tg2d)


def make(name: str, shape=None, **kw) -> Workload:
    fn = WORKLOADS[name]
    return fn(shape, **kw) if shape is not None else fn(**kw)
