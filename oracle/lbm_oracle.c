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
 *  R14 The two-dimensional variant of [TL] Sec. 2 (D2Q9 for the flow, D2Q5
 *      for the temperature) runs on a box with nz = 1 and periodic z faces.
 *      D2Q9 = rest, 4 axis and 4 diagonal vectors of the xy plane with
 *      weights 4/9, 1/9, 1/36; M = the orthogonal basis of Lallemand and Luo
 *      (the 2D member of the d'Humieres family); rows, as polynomials of c:
 *        1, 3c^2-4, (9c^4-21c^2+8)/2, cx, (3c^2-5)cx, cy, (3c^2-5)cy,
 *        cx^2-cy^2, cx cy;
 *      S = diag(s9[0..8]); m_eq = M f_eq and F~ as in R3-R4 with the D2Q9
 *      weights.  [TL] puts the buoyancy along y in 2D; here it is the
 *      vector gbeta, as in R5.
 *  R15 D2Q5, directions ordered (0,+x,-x,+y,-y); N rows (1,1,1,1,1), e_x,
 *      e_y, (-4,1,1,1,1), (0,1,1,-1,-1); n_eq = (T, ux T, uy T, a_T T, 0);
 *      Q = diag(s5[0..4]).  The anti-bounce-back constant is the one [TL]
 *      Sec. 2 gives for D2Q5, w = (4 + a_T)/10.
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
#define Q9 9
#define Q5 5
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
    int32_t lattice;          /* 0: D3Q19 (+ D3Q7), 1: D2Q9 (+ D2Q5) on nz = 1 (R14) */
    int32_t pad1;
    double s9[9];             /* D2Q9 MRT rates in the row order of R14 */
    double s5[5];             /* D2Q5 rates in the row order of R15 */
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
static int C9[Q9][3];
static double W9[Q9];
static int OPP9[Q9];
static double M9[Q9][Q9];
static double MINV9[Q9][Q9];
static int C5[Q5][3];
static int OPP5[Q5];
static double N5[Q5][Q5];
static double NINV5[Q5][Q5];
static int tables_ready = 0;

/* One lattice pair of the double-distribution model: the flow lattice (Q
   velocities C, weights W, moment matrix M) and the temperature lattice (QT
   velocities CT, moment matrix N), plus the anti-bounce-back constant
   w = (wnum + a_T) / wden of [TL] Sec. 2. */
typedef struct lattice {
    int Q;
    const int (*C)[3];
    const double* W;
    const int* OPP;
    const double* M;    /* Q x Q, row k = moment k */
    const double* MINV;
    int QT;
    const int (*CT)[3];
    const int* OPPT;
    const double* N;    /* QT x QT */
    const double* NINV;
    double wnum, wden;
} lattice;

static lattice LAT3, LAT2;

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

/* Moment polynomials of R14 (D2Q9), evaluated at one velocity vector. */
static void moment_row_values_2d(const int* c, double* row)
{
    double cx = c[0], cy = c[1];
    double c2 = cx * cx + cy * cy;
    row[0] = 1.0;
    row[1] = 3.0 * c2 - 4.0;
    row[2] = (9.0 * c2 * c2 - 21.0 * c2 + 8.0) / 2.0;
    row[3] = cx;
    row[4] = (3.0 * c2 - 5.0) * cx;
    row[5] = cy;
    row[6] = (3.0 * c2 - 5.0) * cy;
    row[7] = cx * cx - cy * cy;
    row[8] = cx * cy;
}

/* Every c in {-1,0,1}^dims (z = 0 when dims = 2) with |c|^2 <= 2, rest
   first, then by |c|^2, each vector followed by its opposite; returns the
   count. */
static int velocity_set(int dims, int (*C)[3])
{
    int n = 0;
    int zr = dims == 3 ? 1 : 0;
    for (int len2 = 0; len2 <= 2; ++len2)
        for (int z = -zr; z <= zr; ++z)
            for (int y = -1; y <= 1; ++y)
                for (int x = -1; x <= 1; ++x) {
                    if (x * x + y * y + z * z != len2) continue;
                    /* keep only the "positive" member of each pair here */
                    int first = x != 0 ? x : (y != 0 ? y : z);
                    if (len2 > 0 && first < 0) continue;
                    C[n][0] = x; C[n][1] = y; C[n][2] = z; ++n;
                    if (len2 > 0) { C[n][0] = -x; C[n][1] = -y; C[n][2] = -z; ++n; }
                }
    return n;
}

static int opposites(int Q, const int (*C)[3], int* opp)
{
    for (int q = 0; q < Q; ++q) {
        opp[q] = -1;
        for (int p = 0; p < Q; ++p)
            if (C[p][0] == -C[q][0] && C[p][1] == -C[q][1] && C[p][2] == -C[q][2]) opp[q] = p;
        if (opp[q] < 0) return -1;
    }
    return 0;
}

static int build_tables(void)
{
    if (tables_ready) return 0;
    /* R1 */
    if (velocity_set(3, C19) != Q19) return -1;
    for (int q = 0; q < Q19; ++q) {
        int l2 = C19[q][0] * C19[q][0] + C19[q][1] * C19[q][1] + C19[q][2] * C19[q][2];
        W19[q] = l2 == 0 ? 1.0 / 3.0 : (l2 == 1 ? 1.0 / 18.0 : 1.0 / 36.0);
    }
    if (opposites(Q19, (const int (*)[3])C19, OPP19)) return -1;
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
    if (opposites(Q7, (const int (*)[3])C7, OPP7)) return -1;
    if (invert(Q7, &N7[0][0], &NINV7[0][0])) return -1;

    /* R14: D2Q9 */
    if (velocity_set(2, C9) != Q9) return -1;
    for (int q = 0; q < Q9; ++q) {
        int l2 = C9[q][0] * C9[q][0] + C9[q][1] * C9[q][1];
        W9[q] = l2 == 0 ? 4.0 / 9.0 : (l2 == 1 ? 1.0 / 9.0 : 1.0 / 36.0);
    }
    if (opposites(Q9, (const int (*)[3])C9, OPP9)) return -1;
    double mrow9[Q9];
    for (int q = 0; q < Q9; ++q) {
        moment_row_values_2d(C9[q], mrow9);
        for (int k = 0; k < Q9; ++k) M9[k][q] = mrow9[k];
    }
    if (invert(Q9, &M9[0][0], &MINV9[0][0])) return -1;

    /* R15: D2Q5 */
    static const int c5[Q5][3] = {{0, 0, 0}, {1, 0, 0}, {-1, 0, 0}, {0, 1, 0}, {0, -1, 0}};
    static const double n5[Q5][Q5] = {
        {1, 1, 1, 1, 1},
        {0, 1, -1, 0, 0},
        {0, 0, 0, 1, -1},
        {-4, 1, 1, 1, 1},
        {0, 1, 1, -1, -1}};
    for (int k = 0; k < Q5; ++k) {
        for (int a = 0; a < 3; ++a) C5[k][a] = c5[k][a];
        for (int j = 0; j < Q5; ++j) N5[k][j] = n5[k][j];
    }
    if (opposites(Q5, (const int (*)[3])C5, OPP5)) return -1;
    if (invert(Q5, &N5[0][0], &NINV5[0][0])) return -1;

    LAT3 = (lattice){Q19, (const int (*)[3])C19, W19, OPP19, &M19[0][0], &MINV19[0][0],
                     Q7, (const int (*)[3])C7, OPP7, &N7[0][0], &NINV7[0][0], 6.0, 21.0};
    LAT2 = (lattice){Q9, (const int (*)[3])C9, W9, OPP9, &M9[0][0], &MINV9[0][0],
                     Q5, (const int (*)[3])C5, OPP5, &N5[0][0], &NINV5[0][0], 4.0, 10.0};
    tables_ready = 1;
    return 0;
}

static const lattice* lattice_of(const oracle_params* p) { return p->lattice == 1 ? &LAT2 : &LAT3; }

/* The flow and temperature rates of the lattice in use. */
static const double* flow_rates(const oracle_params* p) { return p->lattice == 1 ? p->s9 : p->s19; }
static const double* temp_rates(const oracle_params* p) { return p->lattice == 1 ? p->s5 : p->s7; }

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

/* The same for the two-dimensional pair (D2Q9, D2Q5). */
int oracle_tables_2d(int32_t* c9, double* w9, int32_t* opp9, double* m9, double* minv9,
                     int32_t* c5, int32_t* opp5, double* n5, double* ninv5)
{
    if (build_tables()) return -1;
    for (int q = 0; q < Q9; ++q) {
        for (int a = 0; a < 3; ++a) c9[q * 3 + a] = C9[q][a];
        w9[q] = W9[q];
        opp9[q] = OPP9[q];
        for (int k = 0; k < Q9; ++k) {
            m9[q * Q9 + k] = M9[q][k];
            minv9[q * Q9 + k] = MINV9[q][k];
        }
    }
    for (int k = 0; k < Q5; ++k) {
        for (int a = 0; a < 3; ++a) c5[k * 3 + a] = C5[k][a];
        opp5[k] = OPP5[k];
        for (int j = 0; j < Q5; ++j) {
            n5[k * Q5 + j] = N5[k][j];
            ninv5[k * Q5 + j] = NINV5[k][j];
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
    const lattice* L = lattice_of(p);
    double rho = 0.0, j[3] = {0.0, 0.0, 0.0};
    for (int q = 0; q < L->Q; ++q) {
        rho += f[q];
        for (int a = 0; a < 3; ++a) j[a] += L->C[q][a] * f[q];
    }
    double T = 0.0;
    if (p->thermal)
        for (int k = 0; k < L->QT; ++k) T += g[k];
    for (int a = 0; a < 3; ++a) {
        F[a] = rho * p->accel[a];
        if (p->thermal) F[a] += rho * p->gbeta[a] * (T - p->T0);
        u[a] = (j[a] + 0.5 * F[a]) / rho;
    }
    *rho_out = rho;
    *T_out = T;
}

static void f_equilibrium(const lattice* L, double rho, const double* u, double* feq)
{
    double uu = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
    for (int q = 0; q < L->Q; ++q) {
        double cu = L->C[q][0] * u[0] + L->C[q][1] * u[1] + L->C[q][2] * u[2];
        feq[q] = L->W[q] * rho * (1.0 + 3.0 * cu + 4.5 * cu * cu - 1.5 * uu);
    }
}

/* R6 (D3Q7) and R15 (D2Q5): (T, u T, a_T T, 0, ...) */
static void g_equilibrium_moments(const oracle_params* p, double T, const double* u, double* neq)
{
    const lattice* L = lattice_of(p);
    int dims = L->QT == Q7 ? 3 : 2;
    for (int k = 0; k < L->QT; ++k) neq[k] = 0.0;
    neq[0] = T;
    for (int a = 0; a < dims; ++a) neq[1 + a] = u[a] * T;
    neq[1 + dims] = p->a_T * T;
}

static void g_from_moments(const lattice* L, const double* n, double* g)
{
    for (int k = 0; k < L->QT; ++k) {
        g[k] = 0.0;
        for (int j = 0; j < L->QT; ++j) g[k] += L->NINV[k * L->QT + j] * n[j];
    }
}

/* One cell's collision ([TL] Eq. 5-7 with the readings R2-R6, R14-R15). */
static void collide_cell(const oracle_params* p, const double* f, const double* g,
                         double* fpost, double* gpost, double* mac)
{
    const lattice* L = lattice_of(p);
    const int Q = L->Q;
    const double* s = flow_rates(p);
    double rho, u[3], T, F[3];
    macros(p, f, g, &rho, u, &T, F);

    double feq[Q19], Ft[Q19];
    f_equilibrium(L, rho, u, feq);
    for (int q = 0; q < Q; ++q) {
        double cu = L->C[q][0] * u[0] + L->C[q][1] * u[1] + L->C[q][2] * u[2];
        double sum = 0.0;
        for (int a = 0; a < 3; ++a) sum += (3.0 * (L->C[q][a] - u[a]) + 9.0 * cu * L->C[q][a]) * F[a];
        Ft[q] = L->W[q] * sum;
    }
    double m[Q19], meq[Q19], mF[Q19], mstar[Q19];
    for (int k = 0; k < Q; ++k) {
        m[k] = meq[k] = mF[k] = 0.0;
        for (int q = 0; q < Q; ++q) {
            m[k] += L->M[k * Q + q] * f[q];
            meq[k] += L->M[k * Q + q] * feq[q];
            mF[k] += L->M[k * Q + q] * Ft[q];
        }
    }
    for (int k = 0; k < Q; ++k)
        mstar[k] = m[k] - s[k] * (m[k] - meq[k]) + (1.0 - 0.5 * s[k]) * mF[k];
    for (int q = 0; q < Q; ++q) {
        fpost[q] = 0.0;
        for (int k = 0; k < Q; ++k) fpost[q] += L->MINV[q * Q + k] * mstar[k];
    }

    if (p->thermal) {
        const int QT = L->QT;
        const double* sT = temp_rates(p);
        double n[Q7], neq[Q7], nstar[Q7];
        g_equilibrium_moments(p, T, u, neq);
        for (int k = 0; k < QT; ++k) {
            n[k] = 0.0;
            for (int j = 0; j < QT; ++j) n[k] += L->N[k * QT + j] * g[j];
        }
        for (int k = 0; k < QT; ++k) nstar[k] = n[k] - sT[k] * (n[k] - neq[k]);
        g_from_moments(L, nstar, gpost);
    }
    if (mac) {
        mac[0] = rho;
        mac[1] = u[0];
        mac[2] = u[1];
        mac[3] = u[2];
        mac[4] = T;
    }
}

/* Collide a batch of cells given as cell-major arrays f[n][Q], g[n][QT]
   (Q, QT those of the lattice in use).  mac[n][5] = (rho, ux, uy, uz, T) of
   the pre-collision state. */
int oracle_collide(const oracle_params* p, int64_t ncells, const double* f, const double* g,
                   double* fpost, double* gpost, double* mac)
{
    if (build_tables() || !p || ncells < 0) return -1;
    if (p->thermal && (!g || !gpost)) return -1;
    const lattice* L = lattice_of(p);
    for (int64_t i = 0; i < ncells; ++i)
        collide_cell(p, f + i * L->Q, p->thermal ? g + i * L->QT : NULL, fpost + i * L->Q,
                     p->thermal ? gpost + i * L->QT : NULL, mac ? mac + i * 5 : NULL);
    return 0;
}

/* Equilibria for a batch of (rho, u, T): feq[n][Q], geq[n][QT] (R7). */
int oracle_equilibrium(const oracle_params* p, int64_t ncells, const double* rho, const double* u,
                       const double* T, double* feq, double* geq)
{
    if (build_tables() || !p) return -1;
    const lattice* L = lattice_of(p);
    for (int64_t i = 0; i < ncells; ++i) {
        double uu[3] = {u[i * 3], u[i * 3 + 1], u[i * 3 + 2]};
        f_equilibrium(L, rho[i], uu, feq + i * L->Q);
        if (geq) {
            double neq[Q7];
            g_equilibrium_moments(p, T ? T[i] : 0.0, uu, neq);
            g_from_moments(L, neq, geq + i * L->QT);
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
    /* R14: the two-dimensional lattices live on one periodic z layer */
    if (p->lattice != 0 && p->lattice != 1) return -1;
    if (p->lattice == 1 && (w.N[2] != 1 || p->face_kind[4] != PERIODIC || p->face_kind[5] != PERIODIC)) return -1;
    const lattice* L = lattice_of(p);
    const int Q = L->Q, QT = L->QT;
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

    double* f = (double*)malloc(sizeof(double) * Q * n);
    double* fp = (double*)malloc(sizeof(double) * Q * n);
    double* g = th ? (double*)malloc(sizeof(double) * QT * n) : NULL;
    double* gp = th ? (double*)malloc(sizeof(double) * QT * n) : NULL;
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
            for (int q = 0; q < Q; ++q) f[q * n + l] = nan;
            if (th) for (int k = 0; k < QT; ++k) g[k * n + l] = nan;
            continue;
        }
        if (f0) {
            for (int q = 0; q < Q; ++q) f[q * n + l] = f0[q * n + l];
            if (th) for (int k = 0; k < QT; ++k) g[k * n + l] = g0[k * n + l];
        } else {
            double uu[3] = {u0[l], u0[n + l], u0[2 * n + l]};
            double feq[Q19];
            f_equilibrium(L, rho0[l], uu, feq);
            for (int q = 0; q < Q; ++q) f[q * n + l] = feq[q];
            if (th) {
                double neq[Q7], geq[Q7];
                g_equilibrium_moments(p, T0[l], uu, neq);
                g_from_moments(L, neq, geq);
                for (int k = 0; k < QT; ++k) g[k * n + l] = geq[k];
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
                for (int q = 0; q < Q; ++q) fp[q * n + l] = nan;
                if (th) for (int k = 0; k < QT; ++k) gp[k * n + l] = nan;
                continue;
            }
            for (int q = 0; q < Q; ++q) fl[q] = f[q * n + l];
            if (th) for (int k = 0; k < QT; ++k) gl[k] = g[k * n + l];
            double mac[5];
            collide_cell(p, fl, th ? gl : NULL, fo, th ? go : NULL, mac);
            for (int a = 0; a < 3; ++a) uc[a * n + l] = mac[1 + a];
            for (int q = 0; q < Q; ++q) fp[q * n + l] = fo[q];
            if (th) for (int k = 0; k < QT; ++k) gp[k * n + l] = go[k];
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
                for (int q = 0; q < Q; ++q) {
                    int o = L->OPP[q];
                    int rule = WALL, axis = 0;
                    int grp = face_rule(p, w.N, gc, L->C[o], &rule, &axis);
                    if (grp < 0) grp = blocked_group(p, labels, w.N, gc, L->C[o]); /* a solid: WALL */
                    if (grp >= 0 && rule == SLIP) {
                        /* R10 SLIP: q arrives from y = x - c_t, sent along q with its normal
                           component reversed (the tangential part c_t of c_q is kept) */
                        int pr = -1, ct[3];
                        for (int a = 0; a < 3; ++a) ct[a] = a == axis ? 0 : L->C[q][a];
                        for (int r = 0; r < Q; ++r)
                            if (L->C[r][axis] == -L->C[q][axis] && L->C[r][(axis + 1) % 3] == L->C[q][(axis + 1) % 3] &&
                                L->C[r][(axis + 2) % 3] == L->C[q][(axis + 2) % 3])
                                pr = r;
                        int64_t src[3];
                        for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - ct[a], w.N[a]);
                        int64_t ls = global_to_local(&w, src);
                        double v = ls >= 0 ? fp[pr * n + ls] : nan;
                        f[q * n + l] = v;
                        if (pd && grp < ngroups)
                            for (int a = 0; a < 3; ++a) pd[grp * 4 + a] += (L->C[pr][a] - L->C[q][a]) * v;
                    } else if (grp >= 0) {
                        /* the population x sent along c_o comes back along c_q (R10) */
                        double v = fp[o * n + l], vin = v;
                        if (rule == VELOCITY) {
                            double cu = 0.0;
                            for (int a = 0; a < 3; ++a) cu += L->C[o][a] * p->face_u[3 * grp + a];
                            vin = v - 6.0 * L->W[o] * p->face_rho[grp] * cu;
                        } else if (rule == PRESSURE) {
                            double cu = 0.0, uu = 0.0;
                            for (int a = 0; a < 3; ++a) {
                                double ua = uc[a * n + l];
                                cu += L->C[o][a] * ua;
                                uu += ua * ua;
                            }
                            vin = -v + 2.0 * L->W[o] * p->face_rho[grp] * (1.0 + 4.5 * cu * cu - 1.5 * uu);
                        }
                        f[q * n + l] = vin;
                        /* R9: momentum out along c_o minus momentum back along c_q = -c_o */
                        if (pd && grp < ngroups)
                            for (int a = 0; a < 3; ++a) pd[grp * 4 + a] += L->C[o][a] * (v + vin);
                    } else {
                        int64_t src[3];
                        for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - L->C[q][a], w.N[a]);
                        int64_t ls = global_to_local(&w, src);
                        f[q * n + l] = ls >= 0 ? fp[q * n + ls] : nan;
                    }
                }
                if (th) {
                    for (int k = 0; k < QT; ++k) {
                        int o = L->OPPT[k];
                        int grp = blocked_group(p, labels, w.N, gc, L->CT[o]);
                        if (grp >= 0) {
                            double v = gp[o * n + l];
                            if (wall_is_dirichlet(p, grp)) {
                                double omega = (L->wnum + p->a_T) / L->wden;
                                double tw = wall_temperature(p, grp);
                                g[k * n + l] = -v + omega * tw;
                                if (pd && grp < ngroups) pd[grp * 4 + 3] += omega * tw - 2.0 * v;
                            } else {
                                g[k * n + l] = v;
                            }
                        } else {
                            int64_t src[3];
                            for (int a = 0; a < 3; ++a) src[a] = wrap_coord(gc[a] - L->CT[k][a], w.N[a]);
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
            for (int q = 0; q < Q; ++q) fl[q] = f[q * n + l];
            if (th) for (int k = 0; k < QT; ++k) gl[k] = g[k * n + l];
            macros(p, fl, th ? gl : NULL, &r, uu, &t, F);
            if (!th) t = 0.0;
        }
        if (rho) rho[l] = r;
        if (u) { u[l] = uu[0]; u[n + l] = uu[1]; u[2 * n + l] = uu[2]; }
        if (T) T[l] = t;
    }
    if (f_out) memcpy(f_out, f, sizeof(double) * Q * n);
    if (g_out && th) memcpy(g_out, g, sizeof(double) * QT * n);

    free(part);
    free(f); free(fp); free(g); free(gp); free(solid); free(uc);
    return 0;
}

/* Velocity-set sizes, for the ctypes wrapper's sanity checks. */
int oracle_q19(void) { return Q19; }
int oracle_q7(void) { return Q7; }
int oracle_q9(void) { return Q9; }
int oracle_q5(void) { return Q5; }
int oracle_max_groups(void) { return MAXGROUPS; }
