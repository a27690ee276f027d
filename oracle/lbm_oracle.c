/*
 * lbm_oracle.c -- plain, slow, fp64 CPU oracle for the fused lattice
 * Boltzmann time step: D3Q19 MRT collision with a Guo-type force term,
 * half-way bounce-back walls, and the double-distribution thermal variant
 * (D3Q7 MRT temperature lattice, anti-bounce-back / bounce-back walls,
 * Boussinesq buoyancy).
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product (the HIP
 * library and its Python binding) never loads it and never falls back to it.
 * It shares no source, header, table or helper with the HIP path.
 *
 * What it follows (page titles and the place on each page):
 *  [KF]  "GPU Optimization for High-Quality Kinetic Fluid Simulation"
 *        (Chen, Li, Fan, Liu), Sec. 3.1, Eq. 1 (lattice Boltzmann update),
 *        Eq. 3 (streaming f*_i(x) = f_i(x - c_i)), Eq. 4 (collide with a
 *        force term), Eq. 5 (MRT relaxation in moment space);
 *        Sec. 4.2, Fig. 6 / Alg. 1 (bounce-back when x - c_i is solid).
 *  [TL]  "Multi-GPU thermal lattice Boltzmann simulations using OpenACC and
 *        MPI", Sec. 2: Eq. 5 (f evolution), the force term
 *        F' = M^-1 (I - S/2) M F~ (Eq. 6), F = rho g beta_T (T - T0) z,
 *        rho = sum f, u = (sum e f + F/2) / rho, half-way bounce-back
 *        f_ibar(x, t+dt) = f_i^+(x, t); Eq. 7 (g evolution), T = sum g,
 *        anti-bounce-back g_ibar(x, t+dt) = -g_i^+(x, t) + w T_w with
 *        w = (6 + a_T)/21 for D3Q7, adiabatic bounce-back
 *        g_ibar = g_i^+; Sec. 3, the split of each evolution equation into a
 *        collision step then a streaming step.
 *  [AA]  "GPU lattice Boltzmann: streaming layout and performance"
 *        (OneCAD-Simulation docs): forces are taken per wall link
 *        (momentum exchange) at the step whose forces are read back.
 *
 * Readings taken where the pages are silent (each one is a choice, not a
 * fact the pages state):
 *  R1  D3Q19 velocity set = rest, 6 axis and 12 face-diagonal vectors with
 *      weights 1/3, 1/18, 1/36 (the page's lattice figure is not available).
 *  R2  M = the orthogonal polynomial moment basis of d'Humieres et al.
 *      (cited by [KF] for RM-MRT); rows, as polynomials of c:
 *        1, 19c^2-30, (21c^4-53c^2+24)/2,
 *        cx, (5c^2-9)cx, cy, (5c^2-9)cy, cz, (5c^2-9)cz,
 *        3cx^2-c^2, (3c^2-5)(3cx^2-c^2), cy^2-cz^2, (3c^2-5)(cy^2-cz^2),
 *        cx cy, cy cz, cx cz,
 *        (cy^2-cz^2)cx, (cz^2-cx^2)cy, (cx^2-cy^2)cz.
 *      S = diag(s19[0..18]) in this row order.  M^-1 is inverted
 *      numerically (Gauss-Jordan), not written out.
 *  R3  m_eq = M f_eq with the second-order equilibrium
 *      f_eq_i = w_i rho [1 + 3 c.u + 9/2 (c.u)^2 - 3/2 u.u].
 *  R4  F~_i = w_i [3 (c_i - u) + 9 (c_i.u) c_i] . F   (Guo's form), so the
 *      force term of [TL] Eq. 6 is M^-1 (I - S/2) M F~.
 *  R5  Force F = rho*accel + rho*gbeta*(T - T0); gbeta is a vector (the
 *      buoyancy direction points against gravity).
 *  R6  D3Q7, directions ordered (0,+x,-x,+y,-y,+z,-z); N rows
 *        (1,1,1,1,1,1,1), e_x, e_y, e_z, (-6,1,1,1,1,1,1),
 *        (0,2,2,-1,-1,-1,-1), (0,0,0,1,1,-1,-1);
 *      n_eq = (T, ux T, uy T, uz T, a_T T, 0, 0);  Q = diag(s7[0..6]).
 *  R7  Initial state: f = f_eq(rho0, u0), g = N^-1 n_eq(T0, u0).
 *  R8  A link (x, p) is blocked when x + c_p leaves the box through a
 *      non-periodic face (group = that face; for a link crossing two faces,
 *      the first crossed axis in x, y, z order) or when the periodic image
 *      of x + c_p is a solid cell (group = 5 + its label).  Faces are
 *      numbered 0..5 = x-, x+, y-, y+, z-, z+.
 *  R9  Momentum exchange on a blocked f link: the boundary receives the
 *      momentum the link carries out minus what it brings back,
 *      c_p f_out - c_in f_in (2 c_p f_p^+ for a wall); heat into the fluid
 *      through a Dirichlet g link: w T_w - 2 g_p^+.
 *  R10 Face kinds ([AA] names wall, reflection and open-face rules as
 *      per-link rules; the pages give no formulas, these are the textbook
 *      half-way forms).  For a link (x, p) that leaves through face f:
 *        WALL      f_pbar(x) = f_p^+(x)                  (no-slip, at rest)
 *        SLIP      specular reflection: the normal part of c_p reverses,
 *                  the tangential part c_t carries on, so the population
 *                  arrives at x + c_t along q = p reflected:
 *                  f_q(x + c_t) = f_p^+(x)               (free slip)
 *        VELOCITY  bounce-back off a wall moving at u_w (Ladd):
 *                  f_pbar(x) = f_p^+(x) - 6 w_p rho_w c_p.u_w
 *                  (a velocity inlet when u_w crosses the face, a moving
 *                  lid when it is tangential)
 *        PRESSURE  anti-bounce-back at density rho_w with the cell's own
 *                  velocity u(x) of that step:
 *                  f_pbar(x) = -f_p^+(x)
 *                              + 2 w_p rho_w [1 + 9/2 (c_p.u)^2 - 3/2 u.u]
 *                  (an open outlet).
 *      rho_w and u_w are per-face parameters.
 *  R11 A link leaving through two faces takes the rule of the first crossed
 *      axis in x, y, z order, with SLIP acting as WALL there (reflecting
 *      both normal components is bounce-back).
 *  R12 The D3Q7 lattice takes each non-periodic face's thermal rule
 *      (Dirichlet anti-bounce-back or adiabatic bounce-back) whatever its
 *      kind; an axis is periodic on both faces or on neither.
 *  R13 No solid cell may lie in the first cell layer of a SLIP face (the
 *      reflected population travels along that layer).
 *
 * Windows: the oracle can run on a window (a sub-box, possibly wrapping
 * through periodic faces) of the full box.  A population that would be
 * pulled from a cell outside the window is set to NaN, so after n steps
 * every cell at Chebyshev distance > n from a cut window edge is exact.
 * A window equal to the whole box is the plain full-domain definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q19 19
#define Q7 7
#define MAXGROUPS 261 /* 6 faces + 255 solid labels */

typedef struct oracle_params {
    int32_t nx, ny, nz;
    int32_t thermal;          /* 0: flow only, 1: flow + D3Q7 temperature */
    int32_t face_kind[6];     /* 0 periodic, 1 wall, 2 slip, 3 velocity, 4 pressure (R10) */
    int32_t face_thermal[6];  /* 0 adiabatic, 1 Dirichlet */
    double face_T[6];         /* Dirichlet wall temperature */
    int32_t solid_thermal;    /* 0 adiabatic, 1 Dirichlet (all solids) */
    int32_t pad0;
    double solid_T;
    double s19[19];           /* MRT rates in the row order of R2 */
    double s7[7];             /* D3Q7 rates in the row order of R6 */
    double a_T;
    double accel[3];
    double gbeta[3];
    double T0;
    double face_u[18];        /* wall velocity u_w of each face (VELOCITY faces) */
    double face_rho[6];       /* wall density rho_w of each face (VELOCITY, PRESSURE) */
} oracle_params;

enum { PERIODIC = 0, WALL = 1, SLIP = 2, VELOCITY = 3, PRESSURE = 4 };

/* ------------------------------------------------------------------ tables */

static int C19[Q19][3];
static double W19[Q19];
static int OPP19[Q19];
static double M19[Q19][Q19];
static double MINV19[Q19][Q19];
static int C7[Q7][3];
static int OPP7[Q7];
static double N7[Q7][Q7];
static double NINV7[Q7][Q7];
static int tables_ready = 0;

/* Gauss-Jordan inversion with partial pivoting; returns 0 on success. */
static int invert(int n, const double* a, double* inv)
{
    double* w = (double*)malloc(sizeof(double) * n * 2 * n);
    if (!w) return -1;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < 2 * n; ++j)
            w[i * 2 * n + j] = j < n ? a[i * n + j] : (j - n == i ? 1.0 : 0.0);
    for (int col = 0; col < n; ++col) {
        int piv = col;
        for (int r = col + 1; r < n; ++r)
            if (fabs(w[r * 2 * n + col]) > fabs(w[piv * 2 * n + col])) piv = r;
        if (fabs(w[piv * 2 * n + col]) < 1e-12) { free(w); return -1; }
        if (piv != col)
            for (int j = 0; j < 2 * n; ++j) {
                double t = w[col * 2 * n + j];
                w[col * 2 * n + j] = w[piv * 2 * n + j];
                w[piv * 2 * n + j] = t;
            }
        double d = w[col * 2 * n + col];
        for (int j = 0; j < 2 * n; ++j) w[col * 2 * n + j] /= d;
        for (int r = 0; r < n; ++r) {
            if (r == col) continue;
            double fct = w[r * 2 * n + col];
            if (fct == 0.0) continue;
            for (int j = 0; j < 2 * n; ++j) w[r * 2 * n + j] -= fct * w[col * 2 * n + j];
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) inv[i * n + j] = w[i * 2 * n + n + j];
    free(w);
    return 0;
}

/* Moment polynomials of R2, evaluated at one velocity vector. */
static void moment_row_values(const int* c, double* row)
{
    double cx = c[0], cy = c[1], cz = c[2];
    double c2 = cx * cx + cy * cy + cz * cz;
    row[0] = 1.0;
    row[1] = 19.0 * c2 - 30.0;
    row[2] = (21.0 * c2 * c2 - 53.0 * c2 + 24.0) / 2.0;
    row[3] = cx;
    row[4] = (5.0 * c2 - 9.0) * cx;
    row[5] = cy;
    row[6] = (5.0 * c2 - 9.0) * cy;
    row[7] = cz;
    row[8] = (5.0 * c2 - 9.0) * cz;
    row[9] = 3.0 * cx * cx - c2;
    row[10] = (3.0 * c2 - 5.0) * (3.0 * cx * cx - c2);
    row[11] = cy * cy - cz * cz;
    row[12] = (3.0 * c2 - 5.0) * (cy * cy - cz * cz);
    row[13] = cx * cy;
    row[14] = cy * cz;
    row[15] = cx * cz;
    row[16] = (cy * cy - cz * cz) * cx;
    row[17] = (cz * cz - cx * cx) * cy;
    row[18] = (cx * cx - cy * cy) * cz;
}

static int build_tables(void)
{
    if (tables_ready) return 0;
    /* R1: every c in {-1,0,1}^3 with |c|^2 <= 2, rest first, then by |c|^2,
       each vector followed by its opposite. */
    int n = 0;
    for (int len2 = 0; len2 <= 2; ++len2)
        for (int z = -1; z <= 1; ++z)
            for (int y = -1; y <= 1; ++y)
                for (int x = -1; x <= 1; ++x) {
                    if (x * x + y * y + z * z != len2) continue;
                    /* keep only the "positive" member of each pair here */
                    int first = x != 0 ? x : (y != 0 ? y : z);
                    if (len2 > 0 && first < 0) continue;
                    C19[n][0] = x; C19[n][1] = y; C19[n][2] = z; ++n;
                    if (len2 > 0) { C19[n][0] = -x; C19[n][1] = -y; C19[n][2] = -z; ++n; }
                }
    if (n != Q19) return -1;
    for (int q = 0; q < Q19; ++q) {
        int l2 = C19[q][0] * C19[q][0] + C19[q][1] * C19[q][1] + C19[q][2] * C19[q][2];
        W19[q] = l2 == 0 ? 1.0 / 3.0 : (l2 == 1 ? 1.0 / 18.0 : 1.0 / 36.0);
        OPP19[q] = -1;
        for (int p = 0; p < Q19; ++p)
            if (C19[p][0] == -C19[q][0] && C19[p][1] == -C19[q][1] && C19[p][2] == -C19[q][2])
                OPP19[q] = p;
        if (OPP19[q] < 0) return -1;
    }
    double mrow[Q19];
    for (int q = 0; q < Q19; ++q) {
        moment_row_values(C19[q], mrow);
        for (int k = 0; k < Q19; ++k) M19[k][q] = mrow[k];
    }
    if (invert(Q19, &M19[0][0], &MINV19[0][0])) return -1;

    /* R6: D3Q7 */
    static const int c7[Q7][3] = {{0, 0, 0}, {1, 0, 0}, {-1, 0, 0}, {0, 1, 0},
                                  {0, -1, 0}, {0, 0, 1}, {0, 0, -1}};
    static const double n7[Q7][Q7] = {
        {1, 1, 1, 1, 1, 1, 1},
        {0, 1, -1, 0, 0, 0, 0},
        {0, 0, 0, 1, -1, 0, 0},
        {0, 0, 0, 0, 0, 1, -1},
        {-6, 1, 1, 1, 1, 1, 1},
        {0, 2, 2, -1, -1, -1, -1},
        {0, 0, 0, 1, 1, -1, -1}};
    for (int k = 0; k < Q7; ++k) {
        for (int a = 0; a < 3; ++a) C7[k][a] = c7[k][a];
        for (int j = 0; j < Q7; ++j) N7[k][j] = n7[k][j];
    }
    for (int k = 0; k < Q7; ++k) {
        OPP7[k] = -1;
        for (int p = 0; p < Q7; ++p)
            if (C7[p][0] == -C7[k][0] && C7[p][1] == -C7[k][1] && C7[p][2] == -C7[k][2]) OPP7[k] = p;
    }
    if (invert(Q7, &N7[0][0], &NINV7[0][0])) return -1;
    tables_ready = 1;
    return 0;
}

/* Export the tables so that tests can pin them against closed forms. */
int oracle_tables(int32_t* c19, double* w19, int32_t* opp19, double* m19, double* minv19,
                  int32_t* c7, int32_t* opp7, double* n7, double* ninv7)
{
    if (build_tables()) return -1;
    for (int q = 0; q < Q19; ++q) {
        for (int a = 0; a < 3; ++a) c19[q * 3 + a] = C19[q][a];
        w19[q] = W19[q];
        opp19[q] = OPP19[q];
        for (int k = 0; k < Q19; ++k) {
            m19[q * Q19 + k] = M19[q][k];
            minv19[q * Q19 + k] = MINV19[q][k];
        }
    }
    for (int k = 0; k < Q7; ++k) {
        for (int a = 0; a < 3; ++a) c7[k * 3 + a] = C7[k][a];
        opp7[k] = OPP7[k];
        for (int j = 0; j < Q7; ++j) {
            n7[k * Q7 + j] = N7[k][j];
            ninv7[k * Q7 + j] = NINV7[k][j];
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- one cell */

/* Macroscopic values of the pre-collision state ([TL] Sec. 2):
   rho = sum f, T = sum g, F = rho accel + rho gbeta (T - T0),
   u = (sum c f + F/2) / rho. */
static void macros(const oracle_params* p, const double* f, const double* g,
                   double* rho_out, double* u, double* T_out, double* F)
{
    double rho = 0.0, j[3] = {0.0, 0.0, 0.0};
    for (int q = 0; q < Q19; ++q) {
        rho += f[q];
        for (int a = 0; a < 3; ++a) j[a] += C19[q][a] * f[q];
    }
    double T = 0.0;
    if (p->thermal)
        for (int k = 0; k < Q7; ++k) T += g[k];
    for (int a = 0; a < 3; ++a) {
        F[a] = rho * p->accel[a];
        if (p->thermal) F[a] += rho * p->gbeta[a] * (T - p->T0);
        u[a] = (j[a] + 0.5 * F[a]) / rho;
    }
    *rho_out = rho;
    *T_out = T;
}

static void f_equilibrium(double rho, const double* u, double* feq)
{
    double uu = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
    for (int q = 0; q < Q19; ++q) {
        double cu = C19[q][0] * u[0] + C19[q][1] * u[1] + C19[q][2] * u[2];
        feq[q] = W19[q] * rho * (1.0 + 3.0 * cu + 4.5 * cu * cu - 1.5 * uu);
    }
}

static void g_equilibrium_moments(const oracle_params* p, double T, const double* u, double* neq)
{
    neq[0] = T;
    neq[1] = u[0] * T;
    neq[2] = u[1] * T;
    neq[3] = u[2] * T;
    neq[4] = p->a_T * T;
    neq[5] = 0.0;
    neq[6] = 0.0;
}

/* One cell's collision ([TL] Eq. 5-7 with the readings R2-R6). */
static void collide_cell(const oracle_params* p, const double* f, const double* g,
                         double* fpost, double* gpost, double* mac)
{
    double rho, u[3], T, F[3];
    macros(p, f, g, &rho, u, &T, F);

    double feq[Q19], Ft[Q19];
    f_equilibrium(rho, u, feq);
    for (int q = 0; q < Q19; ++q) {
        double cu = C19[q][0] * u[0] + C19[q][1] * u[1] + C19[q][2] * u[2];
        double s = 0.0;
        for (int a = 0; a < 3; ++a) s += (3.0 * (C19[q][a] - u[a]) + 9.0 * cu * C19[q][a]) * F[a];
        Ft[q] = W19[q] * s;
    }
    double m[Q19], meq[Q19], mF[Q19], mstar[Q19];
    for (int k = 0; k < Q19; ++k) {
        m[k] = meq[k] = mF[k] = 0.0;
        for (int q = 0; q < Q19; ++q) {
            m[k] += M19[k][q] * f[q];
            meq[k] += M19[k][q] * feq[q];
            mF[k] += M19[k][q] * Ft[q];
        }
    }
    for (int k = 0; k < Q19; ++k)
        mstar[k] = m[k] - p->s19[k] * (m[k] - meq[k]) + (1.0 - 0.5 * p->s19[k]) * mF[k];
    for (int q = 0; q < Q19; ++q) {
        fpost[q] = 0.0;
        for (int k = 0; k < Q19; ++k) fpost[q] += MINV19[q][k] * mstar[k];
    }

    if (p->thermal) {
        double n[Q7], neq[Q7], nstar[Q7];
        g_equilibrium_moments(p, T, u, neq);
        for (int k = 0; k < Q7; ++k) {
            n[k] = 0.0;
            for (int j = 0; j < Q7; ++j) n[k] += N7[k][j] * g[j];
        }
        for (int k = 0; k < Q7; ++k) nstar[k] = n[k] - p->s7[k] * (n[k] - neq[k]);
        for (int k = 0; k < Q7; ++k) {
            gpost[k] = 0.0;
            for (int j = 0; j < Q7; ++j) gpost[k] += NINV7[k][j] * nstar[j];
        }
    }
    if (mac) {
        mac[0] = rho;
        mac[1] = u[0];
        mac[2] = u[1];
        mac[3] = u[2];
        mac[4] = T;
    }
}

/* Collide a batch of cells given as cell-major arrays f[n][19], g[n][7].
   mac[n][5] = (rho, ux, uy, uz, T) of the pre-collision state. */
int oracle_collide(const oracle_params* p, int64_t ncells, const double* f, const double* g,
                   double* fpost, double* gpost, double* mac)
{
    if (build_tables() || !p || ncells < 0) return -1;
    if (p->thermal && (!g || !gpost)) return -1;
    for (int64_t i = 0; i < ncells; ++i)
        collide_cell(p, f + i * Q19, p->thermal ? g + i * Q7 : NULL, fpost + i * Q19,
                     p->thermal ? gpost + i * Q7 : NULL, mac ? mac + i * 5 : NULL);
    return 0;
}

/* Equilibria for a batch of (rho, u, T): feq[n][19], geq[n][7] (R7). */
int oracle_equilibrium(const oracle_params* p, int64_t ncells, const double* rho, const double* u,
                       const double* T, double* feq, double* geq)
{
    if (build_tables() || !p) return -1;
    for (int64_t i = 0; i < ncells; ++i) {
        double uu[3] = {u[i * 3], u[i * 3 + 1], u[i * 3 + 2]};
        f_equilibrium(rho[i], uu, feq + i * Q19);
        if (geq) {
            double neq[Q7];
            g_equilibrium_moments(p, T ? T[i] : 0.0, uu, neq);
            for (int k = 0; k < Q7; ++k) {
                geq[i * Q7 + k] = 0.0;
                for (int j = 0; j < Q7; ++j) geq[i * Q7 + k] += NINV7[k][j] * neq[j];
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------- the domain */

typedef struct window {
    int lo[3], n[3], N[3];
    int64_t cells;
} window;

static int64_t wrap_coord(int64_t v, int N) { return ((v % N) + N) % N; }

/* R8: group of the blocked link from global cell g along c, or -1. */
static int blocked_group(const oracle_params* p, const uint8_t* labels, const int* N,
                         const int64_t* g, const int* c)
{
    int64_t t[3];
    for (int a = 0; a < 3; ++a) {
        t[a] = g[a] + c[a];
        if (t[a] < 0 && p->face_kind[2 * a]) return 2 * a;
        if (t[a] >= N[a] && p->face_kind[2 * a + 1]) return 2 * a + 1;
    }
    if (labels) {
        for (int a = 0; a < 3; ++a) t[a] = wrap_coord(t[a], N[a]);
        uint8_t l = labels[t[0] + (int64_t)N[0] * (t[1] + (int64_t)N[1] * t[2])];
        if (l) return 5 + l;
    }
    return -1;
}

/* R10-R11: group and rule of the link from global cell g along c when it
 * leaves through a face (the solid case is blocked_group's), else -1.  *axis
 * is the axis of the governing face. */
static int face_rule(const oracle_params* p, const int* N, const int64_t* g, const int* c, int* rule,
                     int* axis)
{
    int first = -1, crossed = 0;
    for (int a = 0; a < 3; ++a) {
        int64_t t = g[a] + c[a];
        int f = -1;
        if (t < 0 && p->face_kind[2 * a]) f = 2 * a;
        if (t >= N[a] && p->face_kind[2 * a + 1]) f = 2 * a + 1;
        if (f >= 0) {
            if (first < 0) first = f;
            ++crossed;
        }
    }
    if (first < 0) return -1;
    *rule = p->face_kind[first];
    if (*rule == SLIP && crossed > 1) *rule = WALL;
    *axis = first / 2;
    return first;
}

static int is_solid(const uint8_t* labels, const int* N, const int64_t* g)
{
    return labels && labels[g[0] + (int64_t)N[0] * (g[1] + (int64_t)N[1] * g[2])] != 0;
}

static void local_to_global(const window* w, int64_t l, int64_t* g)
{
    int64_t i = l % w->n[0];
    int64_t r = l / w->n[0];
    int64_t j = r % w->n[1];
    int64_t k = r / w->n[1];
    g[0] = wrap_coord(w->lo[0] + i, w->N[0]);
    g[1] = wrap_coord(w->lo[1] + j, w->N[1]);
    g[2] = wrap_coord(w->lo[2] + k, w->N[2]);
}

/* Local index of a global (already wrapped) cell, or -1 outside the window. */
static int64_t global_to_local(const window* w, const int64_t* g)
{
    int64_t li[3];
    for (int a = 0; a < 3; ++a) {
        li[a] = wrap_coord(g[a] - w->lo[a], w->N[a]);
        if (li[a] >= w->n[a]) return -1;
    }
    return li[0] + (int64_t)w->n[0] * (li[1] + (int64_t)w->n[1] * li[2]);
}

static double wall_temperature(const oracle_params* p, int group)
{
    return group < 6 ? p->face_T[group] : p->solid_T;
}

static int wall_is_dirichlet(const oracle_params* p, int group)
{
    return group < 6 ? p->face_thermal[group] : p->solid_thermal;
}

/*
 * Run nsteps of collide-then-stream ([TL] Sec. 3 split; [KF] Eq. 3-4) on a
 * window of the box.
 *   labels   : nx*ny*nz uint8 (0 fluid, l>0 solid with label l), or NULL
 *   win_lo/n : window origin (global) and extent per axis
 *   rho0,u0,T0 : window-local initial macros (u0 as three planes), T0 may be
 *                NULL when not thermal; ignored if f0 is given
 *   f0, g0   : optional window-local initial populations, SoA [q][cell]
 *   rho,u,T  : window-local macros at the final time (pre-collision), NaN on
 *              solid cells; any may be NULL
 *   f_out, g_out : optional final populations, SoA [q][cell]
 *   diag     : optional nsteps*ngroups*4 doubles: per step and group,
 *              (Fx, Fy, Fz) on the wall/solid and Q into the fluid
 *   nthreads : OpenMP threads (<= 0: library default)
 * Returns 0, or -1 for invalid arguments.
 */
int oracle_run(const oracle_params* p, const uint8_t* labels, const int32_t* win_lo,
               const int32_t* win_n, const double* rho0, const double* u0, const double* T0,
               const double* f0, const double* g0, int32_t nsteps, double* rho, double* u,
               double* T, double* f_out, double* g_out, double* diag, int32_t ngroups,
               int32_t nthreads)
{
    if (build_tables() || !p) return -1;
    window w;
    w.N[0] = p->nx; w.N[1] = p->ny; w.N[2] = p->nz;
    for (int a = 0; a < 3; ++a) {
        if (w.N[a] <= 0 || win_n[a] <= 0 || win_n[a] > w.N[a] || win_lo[a] < 0 || win_lo[a] >= w.N[a])
            return -1;
        for (int f = 2 * a; f <= 2 * a + 1; ++f)
            if (p->face_kind[f] < PERIODIC || p->face_kind[f] > PRESSURE) return -1;
        if ((p->face_kind[2 * a] == PERIODIC) != (p->face_kind[2 * a + 1] == PERIODIC)) return -1;
        w.lo[a] = win_lo[a];
        w.n[a] = win_n[a];
    }
    if (nsteps < 0) return -1;
    if (diag && ngroups < 6) return -1;
    /* R13: the first layer of a slip face holds no solid */
    if (labels) {
        for (int f = 0; f < 6; ++f) {
            if (p->face_kind[f] != SLIP) continue;
            const int a = f / 2;
            const int64_t layer = (f & 1) ? w.N[a] - 1 : 0;
            for (int64_t k = 0; k < w.N[2]; ++k)
                for (int64_t j = 0; j < w.N[1]; ++j)
                    for (int64_t i = 0; i < w.N[0]; ++i) {
                        const int64_t gc[3] = {i, j, k};
                        if (gc[a] == layer && is_solid(labels, w.N, gc)) return -1;
                    }
        }
    }
    w.cells = (int64_t)w.n[0] * w.n[1] * w.n[2];
    const int64_t n = w.cells;
    const int th = p->thermal;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    double* f = (double*)malloc(sizeof(double) * Q19 * n);
    double* fp = (double*)malloc(sizeof(double) * Q19 * n);
    double* g = th ? (double*)malloc(sizeof(double) * Q7 * n) : NULL;
    double* gp = th ? (double*)malloc(sizeof(double) * Q7 * n) : NULL;
    uint8_t* solid = (uint8_t*)malloc(n);
    double* uc = (double*)malloc(sizeof(double) * 3 * n); /* each cell's velocity in its last collision */
    if (!f || !fp || (th && (!g || !gp)) || !solid || !uc) {
        free(f); free(fp); free(g); free(gp); free(solid); free(uc);
        return -1;
    }
    const double nan = NAN;

    /* initial state (R7) */
    for (int64_t l = 0; l < n; ++l) {
        int64_t gc[3];
        local_to_global(&w, l, gc);
        solid[l] = (uint8_t)is_solid(labels, w.N, gc);
        if (solid[l]) {
            for (int q = 0; q < Q19; ++q) f[q * n + l] = nan;
            if (th) for (int k = 0; k < Q7; ++k) g[k * n + l] = nan;
            continue;
        }
        if (f0) {
            for (int q = 0; q < Q19; ++q) f[q * n + l] = f0[q * n + l];
            if (th) for (int k = 0; k < Q7; ++k) g[k * n + l] = g0[k * n + l];
        } else {
            double uu[3] = {u0[l], u0[n + l], u0[2 * n + l]};
            double feq[Q19];
            f_equilibrium(rho0[l], uu, feq);
            for (int q = 0; q < Q19; ++q) f[q * n + l] = feq[q];
            if (th) {
                double neq[Q7];
                g_equilibrium_moments(p, T0[l], uu, neq);
                for (int k = 0; k < Q7; ++k) {
                    double s = 0.0;
                    for (int j = 0; j < Q7; ++j) s += NINV7[k][j] * neq[j];
                    g[k * n + l] = s;
                }
            }
        }
    }

    /* per-plane diagnostic partials, summed in plane order (deterministic) */
    double* part = NULL;
    if (diag) {
        part = (double*)calloc((size_t)w.n[2] * ngroups * 4, sizeof(double));
        if (!part) { free(f); free(fp); free(g); free(gp); free(solid); free(uc); return -1; }
    }
    const int64_t plane = (int64_t)w.n[0] * w.n[1];

    for (int step = 0; step < nsteps; ++step) {
        /* collision of every fluid cell of the window */
#pragma omp parallel for schedule(static)
        for (int64_t l = 0; l < n; ++l) {
            double fl[Q19], gl[Q7], fo[Q19], go[Q7];
            if (solid[l]) {
                for (int q = 0; q < Q19; ++q) fp[q * n + l] = nan;
                if (th) for (int k = 0; k < Q7; ++k) gp[k * n + l] = nan;
                continue;
            }
            for (int q = 0; q < Q19; ++q) fl[q] = f[q * n + l];
            if (th) for (int k = 0; k < Q7; ++k) gl[k] = g[k * n + l];
            double mac[5];
            collide_cell(p, fl, th ? gl : NULL, fo, th ? go : NULL, mac);
            for (int a = 0; a < 3; ++a) uc[a * n + l] = mac[1 + a];
            for (int q = 0; q < Q19; ++q) fp[q * n + l] = fo[q];
            if (th) for (int k = 0; k < Q7; ++k) gp[k * n + l] = go[k];
        }
        if (part) memset(part, 0, sizeof(double) * (size_t)w.n[2] * ngroups * 4);

        /* streaming (pull) with half-way bounce-back / anti-bounce-back */
#pragma omp parallel for schedule(static)
        for (int kz = 0; kz < w.n[2]; ++kz) {
            double* pd = part ? part + (size_t)kz * ngroups * 4 : NULL;
            for (int64_t l = kz * plane; l < (kz + 1) * plane; ++l) {
                if (solid[l]) continue;
                int64_t gc[3];
                local_to_global(&w, l, gc);
                for (int q = 0; q < Q19; ++q) {
                    int o = OPP19[q];
                    int rule = WALL, axis = 0;
                    int grp = face_rule(p, w.N, gc, C19[o], &rule, &axis);
                    if (grp < 0) grp = blocked_group(p, labels, w.N, gc, C19[o]); /* a solid: WALL */
                    if (grp >= 0 && rule == SLIP) {
                        /* R10 SLIP: q arrives from y = x - c_t, sent along q with its normal
                           component reversed (the tangential part c_t of c_q is kept) */
                        int pr = -1, ct[3];
                        for (int a = 0; a < 3; ++a) ct[a] = a == axis ? 0 : C19[q][a];
                        for (int r = 0; r < Q19; ++r)
                            if (C19[r][axis] == -C19[q][axis] && C19[r][(axis + 1) % 3] == C19[q][(axis + 1) % 3] &&
                                C19[r][(axis + 2) % 3] == C19[q][(axis + 2) % 3])
                                pr = r;
                        int64_t src[3];
                        for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - ct[a], w.N[a]);
                        int64_t ls = global_to_local(&w, src);
                        double v = ls >= 0 ? fp[pr * n + ls] : nan;
                        f[q * n + l] = v;
                        if (pd && grp < ngroups)
                            for (int a = 0; a < 3; ++a) pd[grp * 4 + a] += (C19[pr][a] - C19[q][a]) * v;
                    } else if (grp >= 0) {
                        /* the population x sent along c_o comes back along c_q (R10) */
                        double v = fp[o * n + l], vin = v;
                        if (rule == VELOCITY) {
                            double cu = 0.0;
                            for (int a = 0; a < 3; ++a) cu += C19[o][a] * p->face_u[3 * grp + a];
                            vin = v - 6.0 * W19[o] * p->face_rho[grp] * cu;
                        } else if (rule == PRESSURE) {
                            double cu = 0.0, uu = 0.0;
                            for (int a = 0; a < 3; ++a) {
                                double ua = uc[a * n + l];
                                cu += C19[o][a] * ua;
                                uu += ua * ua;
                            }
                            vin = -v + 2.0 * W19[o] * p->face_rho[grp] * (1.0 + 4.5 * cu * cu - 1.5 * uu);
                        }
                        f[q * n + l] = vin;
                        /* R9: momentum out along c_o minus momentum back along c_q = -c_o */
                        if (pd && grp < ngroups)
                            for (int a = 0; a < 3; ++a) pd[grp * 4 + a] += C19[o][a] * (v + vin);
                    } else {
                        int64_t src[3];
                        for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - C19[q][a], w.N[a]);
                        int64_t ls = global_to_local(&w, src);
                        f[q * n + l] = ls >= 0 ? fp[q * n + ls] : nan;
                    }
                }
                if (th) {
                    for (int k = 0; k < Q7; ++k) {
                        int o = OPP7[k];
                        int grp = blocked_group(p, labels, w.N, gc, C7[o]);
                        if (grp >= 0) {
                            double v = gp[o * n + l];
                            if (wall_is_dirichlet(p, grp)) {
                                double omega = (6.0 + p->a_T) / 21.0;
                                double tw = wall_temperature(p, grp);
                                g[k * n + l] = -v + omega * tw;
                                if (pd && grp < ngroups) pd[grp * 4 + 3] += omega * tw - 2.0 * v;
                            } else {
                                g[k * n + l] = v;
                            }
                        } else {
                            int64_t src[3];
                            for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - C7[k][a], w.N[a]);
                            int64_t ls = global_to_local(&w, src);
                            g[k * n + l] = ls >= 0 ? gp[k * n + ls] : nan;
                        }
                    }
                }
            }
        }
        if (diag) {
            double* d = diag + (size_t)step * ngroups * 4;
            for (int i = 0; i < ngroups * 4; ++i) d[i] = 0.0;
            for (int kz = 0; kz < w.n[2]; ++kz)
                for (int i = 0; i < ngroups * 4; ++i) d[i] += part[(size_t)kz * ngroups * 4 + i];
        }
    }

    /* outputs */
    for (int64_t l = 0; l < n; ++l) {
        double r = nan, uu[3] = {nan, nan, nan}, t = nan, F[3];
        if (!solid[l]) {
            double fl[Q19], gl[Q7];
            for (int q = 0; q < Q19; ++q) fl[q] = f[q * n + l];
            if (th) for (int k = 0; k < Q7; ++k) gl[k] = g[k * n + l];
            macros(p, fl, th ? gl : NULL, &r, uu, &t, F);
            if (!th) t = 0.0;
        }
        if (rho) rho[l] = r;
        if (u) { u[l] = uu[0]; u[n + l] = uu[1]; u[2 * n + l] = uu[2]; }
        if (T) T[l] = t;
    }
    if (f_out) memcpy(f_out, f, sizeof(double) * Q19 * n);
    if (g_out && th) memcpy(g_out, g, sizeof(double) * Q7 * n);

    free(part);
    free(f); free(fp); free(g); free(gp); free(solid); free(uc);
    return 0;
}

/* Velocity-set sizes, for the ctypes wrapper's sanity checks. */
int oracle_q19(void) { return Q19; }
int oracle_q7(void) { return Q7; }
int oracle_max_groups(void) { return MAXGROUPS; }
