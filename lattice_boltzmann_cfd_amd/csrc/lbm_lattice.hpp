// lbm_lattice.hpp -- per-cell arithmetic of the fused step, kept in registers.
//
// D3Q19 MRT collision with Guo forcing and D3Q7 MRT thermal collision,
// hand-expanded in moment space (no matrices, no MFMA: this is a
// bandwidth-bound stencil, the arithmetic is ~300 flops per cell).
//
// Follows: "Multi-GPU thermal lattice Boltzmann simulations using OpenACC and
// MPI", Sec. 2 -- MRT evolution of f (Eq. 5) with the force term
// F' = M^-1 (I - S/2) M F~ (Eq. 6 and text), rho = sum f,
// u = (sum e f + F/2)/rho, F = rho g beta_T (T - T0) z; MRT evolution of g
// (Eq. 7), T = sum g.  "GPU Optimization for High-Quality Kinetic Fluid
// Simulation", Sec. 3.1, Eq. 5: Omega = -M^-1 D (m - m_eq).  Moment basis,
// equilibria and rates are the readings stated in include/lbm.h.
//
// Storage is shifted: a D3Q19 slot holds h_q = f_q - w_q (the rest-state
// weight removed) so that fp32 keeps the small deviations of f from the rest
// state to full precision.  Moments are computed on h; the weights contribute
// only to rho (1), e (-11) and eps (3), which are folded in analytically.
//
// Direction order of the kernels (their own; not an interface):
//   0 rest; 1 +x, 2 -x, 3 +y, 4 -y, 5 +z, 6 -z;
//   7 (+,+,0)  8 (-,-,0)  9 (+,-,0) 10 (-,+,0)
//  11 (+,0,+) 12 (-,0,-) 13 (+,0,-) 14 (-,0,+)
//  15 (0,+,+) 16 (0,-,-) 17 (0,+,-) 18 (0,-,+)
// D3Q7: 0 rest, 1 +x, 2 -x, 3 +y, 4 -y, 5 +z, 6 -z.
//
// The two-dimensional variant of the same page (D2Q9 flow + D2Q5
// temperature, MRT on both) runs on one periodic z layer.  D2Q9 moment basis
// (Lallemand and Luo; row order of lbm_params.s9): 1, 3c^2-4,
// (9c^4-21c^2+8)/2, cx, (3c^2-5)cx, cy, (3c^2-5)cy, cx^2-cy^2, cx cy, squared
// norms 9, 36, 36, 6, 12, 6, 12, 4, 4.  D2Q5 rows (order of lbm_params.s5):
// 1, e_x, e_y, (-4,1,1,1,1), (0,1,1,-1,-1); n_eq = (T, ux T, uy T, a_T T, 0).
// Direction order of the 2D kernels:
//   D2Q9: 0 rest; 1 +x, 2 -x, 3 +y, 4 -y; 5 (+,+) 6 (-,-) 7 (+,-) 8 (-,+)
//   D2Q5: 0 rest, 1 +x, 2 -x, 3 +y, 4 -y.
// Opposite directions are adjacent pairs (1,2), (3,4), ... in every lattice.
#pragma once

#include <hip/hip_runtime.h>

namespace lbm {

constexpr int Q19 = 19;
constexpr int Q7 = 7;
constexpr int Q9 = 9;
constexpr int Q5 = 5;

__host__ __device__ constexpr int cx19(int q)
{
    constexpr int v[19] = {0, 1, -1, 0, 0, 0, 0, 1, -1, 1, -1, 1, -1, 1, -1, 0, 0, 0, 0};
    return v[q];
}
__host__ __device__ constexpr int cy19(int q)
{
    constexpr int v[19] = {0, 0, 0, 1, -1, 0, 0, 1, -1, -1, 1, 0, 0, 0, 0, 1, -1, 1, -1};
    return v[q];
}
__host__ __device__ constexpr int cz19(int q)
{
    constexpr int v[19] = {0, 0, 0, 0, 0, 1, -1, 0, 0, 0, 0, 1, -1, -1, 1, 1, -1, -1, 1};
    return v[q];
}
// opposite directions come in adjacent pairs (1,2), (3,4), ..., (17,18)
__host__ __device__ constexpr int opp19(int q) { return q == 0 ? 0 : ((q & 1) ? q + 1 : q - 1); }
__host__ __device__ constexpr double w19(int q) { return q == 0 ? 1.0 / 3.0 : (q <= 6 ? 1.0 / 18.0 : 1.0 / 36.0); }

__host__ __device__ constexpr int cx7(int k) { return k == 1 ? 1 : (k == 2 ? -1 : 0); }
__host__ __device__ constexpr int cy7(int k) { return k == 3 ? 1 : (k == 4 ? -1 : 0); }
__host__ __device__ constexpr int cz7(int k) { return k == 5 ? 1 : (k == 6 ? -1 : 0); }
__host__ __device__ constexpr int opp7(int k) { return k == 0 ? 0 : ((k & 1) ? k + 1 : k - 1); }

__host__ __device__ constexpr int cx9(int q)
{
    constexpr int v[9] = {0, 1, -1, 0, 0, 1, -1, 1, -1};
    return v[q];
}
__host__ __device__ constexpr int cy9(int q)
{
    constexpr int v[9] = {0, 0, 0, 1, -1, 1, -1, -1, 1};
    return v[q];
}
__host__ __device__ constexpr double w9(int q) { return q == 0 ? 4.0 / 9.0 : (q <= 4 ? 1.0 / 9.0 : 1.0 / 36.0); }

// The lattice pairs of the double-distribution model as compile-time
// descriptors: flow lattice (Q velocities, weights), temperature lattice (QT
// velocities), spatial dimensions, and the anti-bounce-back constant
// w = (omega_num + a_T) / omega_den of the temperature lattice.
struct Lat3D {
    static constexpr int Q = Q19, QT = Q7, DIMS = 3;
    static constexpr double omega_num = 6.0, omega_den = 21.0;
    __host__ __device__ static constexpr int cx(int q) { return cx19(q); }
    __host__ __device__ static constexpr int cy(int q) { return cy19(q); }
    __host__ __device__ static constexpr int cz(int q) { return cz19(q); }
    __host__ __device__ static constexpr double w(int q) { return w19(q); }
    __host__ __device__ static constexpr int cxT(int k) { return cx7(k); }
    __host__ __device__ static constexpr int cyT(int k) { return cy7(k); }
    __host__ __device__ static constexpr int czT(int k) { return cz7(k); }
};
struct Lat2D {
    static constexpr int Q = Q9, QT = Q5, DIMS = 2;
    static constexpr double omega_num = 4.0, omega_den = 10.0;
    __host__ __device__ static constexpr int cx(int q) { return cx9(q); }
    __host__ __device__ static constexpr int cy(int q) { return cy9(q); }
    __host__ __device__ static constexpr int cz(int) { return 0; }
    __host__ __device__ static constexpr double w(int q) { return w9(q); }
    __host__ __device__ static constexpr int cxT(int k) { return cx7(k); }
    __host__ __device__ static constexpr int cyT(int k) { return cy7(k); }
    __host__ __device__ static constexpr int czT(int) { return 0; }
};
// opposite of direction q in either lattice (adjacent pairs)
__host__ __device__ constexpr int opp(int q) { return q == 0 ? 0 : ((q & 1) ? q + 1 : q - 1); }

// Per-launch constants of the collision (rates and forcing), in the working
// precision R.  Rates of the conserved rows (rho, j) are not needed: their
// post-collision values are rho and j + F for any rate.  The D2Q9 / D2Q5
// rates come last so that the 3D kernels' argument offsets do not depend on
// them.
template <typename R>
struct Collision {
    R s_e, s_eps, s_qx, s_qy, s_qz;
    R s_3pxx, s_3pixx, s_pww, s_piww, s_pxy, s_pyz, s_pxz, s_mx, s_my, s_mz;
    R q_jx, q_jy, q_jz, q_e, q_5, q_6;  // D3Q7 rates (rows 1..6)
    R accel[3];
    R gbeta[3];
    R T0;
    R a_T;
    R s2_e, s2_eps, s2_qx, s2_qy, s2_pxx, s2_pxy;  // D2Q9 rates (rows 1, 2, 4, 6, 7, 8)
    R q2_jx, q2_jy, q2_e, q2_4;                    // D2Q5 rates (rows 1..4)
};

// Macroscopic values of a cell from shifted populations (pre-collision).
template <typename R>
struct Macro {
    R rho, ux, uy, uz, T;
};

// Density deviation, momentum and velocity of the shifted D3Q19 populations h,
// plus T when thermal.  u = j/rho + acc/2 with acc = F/rho.
template <typename R, bool TH>
__device__ __forceinline__ Macro<R> macros(const R (&h)[Q19], const R (&g)[Q7], const Collision<R>& c)
{
    R drho = h[0];
#pragma unroll
    for (int q = 1; q < Q19; ++q) drho += h[q];
    R jx = (h[1] - h[2]) + (h[7] - h[8]) + (h[9] - h[10]) + (h[11] - h[12]) + (h[13] - h[14]);
    R jy = (h[3] - h[4]) + (h[7] - h[8]) - (h[9] - h[10]) + (h[15] - h[16]) + (h[17] - h[18]);
    R jz = (h[5] - h[6]) + (h[11] - h[12]) - (h[13] - h[14]) + (h[15] - h[16]) - (h[17] - h[18]);
    Macro<R> m;
    m.rho = R(1) + drho;
    m.T = R(0);
    R ax = c.accel[0], ay = c.accel[1], az = c.accel[2];
    if (TH) {
        R T = g[0];
#pragma unroll
        for (int k = 1; k < Q7; ++k) T += g[k];
        m.T = T;
        R dT = T - c.T0;
        ax += c.gbeta[0] * dT;
        ay += c.gbeta[1] * dT;
        az += c.gbeta[2] * dT;
    }
    R ir = R(1) / m.rho;
    m.ux = jx * ir + R(0.5) * ax;
    m.uy = jy * ir + R(0.5) * ay;
    m.uz = jz * ir + R(0.5) * az;
    return m;
}

// One cell's collision, in place on the register arrays h (shifted D3Q19) and
// g (D3Q7).  Post-collision = pre-collision + M^-1 dm where, per row k,
// dm_k = -s_k (m_k - m_eq_k) + (1 - s_k/2) (M F~)_k, and dm = 0 (rho) and
// F (j) on the conserved rows.  M^-1 = M^T diag(1/|row|^2) (orthogonal rows).
template <typename R, bool TH>
__device__ __forceinline__ void collide(R (&h)[Q19], R (&g)[Q7], const Collision<R>& c)
{
    // pair sums and differences
    const R sx = h[1] + h[2], dx = h[1] - h[2];
    const R sy = h[3] + h[4], dy = h[3] - h[4];
    const R sz = h[5] + h[6], dz = h[5] - h[6];
    const R a78 = h[7] + h[8], d78 = h[7] - h[8];
    const R a910 = h[9] + h[10], d910 = h[9] - h[10];
    const R a1112 = h[11] + h[12], d1112 = h[11] - h[12];
    const R a1314 = h[13] + h[14], d1314 = h[13] - h[14];
    const R a1516 = h[15] + h[16], d1516 = h[15] - h[16];
    const R a1718 = h[17] + h[18], d1718 = h[17] - h[18];
    const R Sxy = a78 + a910, Dxy = a78 - a910;
    const R Sxz = a1112 + a1314, Dxz = a1112 - a1314;
    const R Syz = a1516 + a1718, Dyz = a1516 - a1718;
    const R Sax = sx + sy + sz;
    const R Sdg = Sxy + Sxz + Syz;
    const R drho = h[0] + Sax + Sdg;
    const R jx = dx + (d78 + d910) + (d1112 + d1314);
    const R jy = dy + (d78 - d910) + (d1516 + d1718);
    const R jz = dz + (d1112 - d1314) + (d1516 - d1718);

    const R rho = R(1) + drho;
    R ax = c.accel[0], ay = c.accel[1], az = c.accel[2];
    R T = R(0);
    if (TH) {
        T = ((g[0] + g[1]) + (g[2] + g[3])) + ((g[4] + g[5]) + g[6]);
        const R dT = T - c.T0;
        ax += c.gbeta[0] * dT;
        ay += c.gbeta[1] * dT;
        az += c.gbeta[2] * dT;
    }
    const R ir = R(1) / rho;
    const R ux = jx * ir + R(0.5) * ax;
    const R uy = jy * ir + R(0.5) * ay;
    const R uz = jz * ir + R(0.5) * az;
    const R Fx = rho * ax, Fy = rho * ay, Fz = rho * az;

    const R uxx = ux * ux, uyy = uy * uy, uzz = uz * uz;
    const R uu = uxx + uyy + uzz;
    const R rdxx = rho * (R(2) * uxx - uyy - uzz);  // rho (2ux^2 - uy^2 - uz^2)
    const R rdww = rho * (uyy - uzz);
    const R uF = ux * Fx + uy * Fy + uz * Fz;
    const R fxx = R(2) * ux * Fx - uy * Fy - uz * Fz;
    const R fww = uy * Fy - uz * Fz;

    // non-equilibrium parts m - m_eq of the shifted moments
    const R ne_e = (R(-30) * h[0] - R(11) * Sax + R(8) * Sdg) + R(11) * drho - R(19) * rho * uu;
    const R ne_eps = (R(12) * h[0] - R(4) * Sax + Sdg) - R(3) * drho + R(5.5) * rho * uu;
    const R two3 = R(2) / R(3);
    const R ne_qx = (jx - R(5) * dx) + two3 * rho * ux;
    const R ne_qy = (jy - R(5) * dy) + two3 * rho * uy;
    const R ne_qz = (jz - R(5) * dz) + two3 * rho * uz;
    const R m3pxx = R(2) * sx - sy - sz + Sxy + Sxz - R(2) * Syz;
    const R m3pixx = R(-4) * sx + R(2) * sy + R(2) * sz + Sxy + Sxz - R(2) * Syz;
    const R mpww = sy - sz + Sxy - Sxz;
    const R mpiww = R(-2) * sy + R(2) * sz + Sxy - Sxz;
    const R ne_3pxx = m3pxx - rdxx;
    const R ne_3pixx = m3pixx + R(0.5) * rdxx;
    const R ne_pww = mpww - rdww;
    const R ne_piww = mpiww + R(0.5) * rdww;
    const R ne_pxy = Dxy - rho * ux * uy;
    const R ne_pyz = Dyz - rho * uy * uz;
    const R ne_pxz = Dxz - rho * ux * uz;
    const R ne_mx = (d78 + d910) - (d1112 + d1314);
    const R ne_my = (d1516 + d1718) - (d78 - d910);
    const R ne_mz = (d1112 - d1314) - (d1516 - d1718);

    // dm_k = -s_k ne_k + (1 - s_k/2) mF_k, divided by the row's squared norm
    const R E = (-c.s_e * ne_e + (R(1) - R(0.5) * c.s_e) * (R(38) * uF)) * R(1.0 / 2394.0);
    const R P = (-c.s_eps * ne_eps + (R(1) - R(0.5) * c.s_eps) * (R(-11) * uF)) * R(1.0 / 252.0);
    const R X = Fx * R(0.1), Y = Fy * R(0.1), Z = Fz * R(0.1);
    const R QX = (-c.s_qx * ne_qx + (R(1) - R(0.5) * c.s_qx) * (-two3 * Fx)) * R(1.0 / 40.0);
    const R QY = (-c.s_qy * ne_qy + (R(1) - R(0.5) * c.s_qy) * (-two3 * Fy)) * R(1.0 / 40.0);
    const R QZ = (-c.s_qz * ne_qz + (R(1) - R(0.5) * c.s_qz) * (-two3 * Fz)) * R(1.0 / 40.0);
    const R A = (-c.s_3pxx * ne_3pxx + (R(1) - R(0.5) * c.s_3pxx) * (R(2) * fxx)) * R(1.0 / 36.0);
    const R B = (-c.s_3pixx * ne_3pixx + (R(1) - R(0.5) * c.s_3pixx) * (-fxx)) * R(1.0 / 72.0);
    const R Cw = (-c.s_pww * ne_pww + (R(1) - R(0.5) * c.s_pww) * (R(2) * fww)) * R(1.0 / 12.0);
    const R Dw = (-c.s_piww * ne_piww + (R(1) - R(0.5) * c.s_piww) * (-fww)) * R(1.0 / 24.0);
    const R Pxy = (-c.s_pxy * ne_pxy + (R(1) - R(0.5) * c.s_pxy) * (ux * Fy + uy * Fx)) * R(0.25);
    const R Pyz = (-c.s_pyz * ne_pyz + (R(1) - R(0.5) * c.s_pyz) * (uy * Fz + uz * Fy)) * R(0.25);
    const R Pxz = (-c.s_pxz * ne_pxz + (R(1) - R(0.5) * c.s_pxz) * (ux * Fz + uz * Fx)) * R(0.25);
    const R MX = -c.s_mx * ne_mx * R(0.125);
    const R MY = -c.s_my * ne_my * R(0.125);
    const R MZ = -c.s_mz * ne_mz * R(0.125);

    // back-transform: f_q += sum_k M[k][q] dm_k / |row k|^2
    const R axisc = R(-11) * E - R(4) * P;
    const R diagc = R(8) * E + P;
    const R XQ = X - R(4) * QX, YQ = Y - R(4) * QY, ZQ = Z - R(4) * QZ;  // axis flux terms
    const R xq = X + QX, yq = Y + QY, zq = Z + QZ;                      // diagonal flux terms
    const R tx = axisc + R(2) * A - R(4) * B;
    const R ty = axisc - A + R(2) * B + Cw - R(2) * Dw;
    const R tz = axisc - A + R(2) * B - Cw + R(2) * Dw;
    const R txy = diagc + A + B + Cw + Dw;
    const R txz = diagc + A + B - Cw - Dw;
    const R tyz = diagc - R(2) * A - R(2) * B;

    h[0] += R(-30) * E + R(12) * P;
    h[1] += tx + XQ;
    h[2] += tx - XQ;
    h[3] += ty + YQ;
    h[4] += ty - YQ;
    h[5] += tz + ZQ;
    h[6] += tz - ZQ;
    h[7] += txy + Pxy + (xq + yq) + (MX - MY);
    h[8] += txy + Pxy - (xq + yq) - (MX - MY);
    h[9] += txy - Pxy + (xq - yq) + (MX + MY);
    h[10] += txy - Pxy - (xq - yq) - (MX + MY);
    h[11] += txz + Pxz + (xq + zq) + (MZ - MX);
    h[12] += txz + Pxz - (xq + zq) - (MZ - MX);
    h[13] += txz - Pxz + (xq - zq) - (MX + MZ);
    h[14] += txz - Pxz - (xq - zq) + (MX + MZ);
    h[15] += tyz + Pyz + (yq + zq) + (MY - MZ);
    h[16] += tyz + Pyz - (yq + zq) - (MY - MZ);
    h[17] += tyz - Pyz + (yq - zq) + (MY + MZ);
    h[18] += tyz - Pyz - (yq - zq) - (MY + MZ);

    if (TH) {
        // D3Q7: n = N g; dn_k = -q_k (n_k - n_eq_k); g += N^T diag(1/|row|^2) dn
        const R n1 = g[1] - g[2], n2 = g[3] - g[4], n3 = g[5] - g[6];
        const R px = g[1] + g[2], py = g[3] + g[4], pz = g[5] + g[6];
        const R n4 = R(-6) * g[0] + (px + py + pz);
        const R n5 = R(2) * px - py - pz;
        const R n6 = py - pz;
        const R K1 = -c.q_jx * (n1 - ux * T) * R(0.5);
        const R K2 = -c.q_jy * (n2 - uy * T) * R(0.5);
        const R K3 = -c.q_jz * (n3 - uz * T) * R(0.5);
        const R K4 = -c.q_e * (n4 - c.a_T * T) * R(1.0 / 42.0);
        const R K5 = -c.q_5 * n5 * R(1.0 / 12.0);
        const R K6 = -c.q_6 * n6 * R(0.25);
        const R bx = K4 + R(2) * K5;
        const R by = K4 - K5 + K6;
        const R bz = K4 - K5 - K6;
        g[0] += R(-6) * K4;
        g[1] += bx + K1;
        g[2] += bx - K1;
        g[3] += by + K2;
        g[4] += by - K2;
        g[5] += bz + K3;
        g[6] += bz - K3;
    }
}

// Shifted equilibrium h_q = f_eq_q - w_q and g_eq for (rho, u, T).
template <typename R, bool TH>
__device__ __forceinline__ void equilibrium(R rho, R ux, R uy, R uz, R T, R a_T, R (&h)[Q19], R (&g)[Q7])
{
    const R uu = ux * ux + uy * uy + uz * uz;
    const R drho = rho - R(1);
#pragma unroll
    for (int q = 0; q < Q19; ++q) {
        const R cu = R(cx19(q)) * ux + R(cy19(q)) * uy + R(cz19(q)) * uz;
        h[q] = R(w19(q)) * (drho + rho * (R(3) * cu + R(4.5) * cu * cu - R(1.5) * uu));
    }
    if (TH) {
        const R wm = (R(6) + a_T) / R(42);
        g[0] = (R(1) - a_T) / R(7) * T;
        g[1] = wm * T + R(0.5) * ux * T;
        g[2] = wm * T - R(0.5) * ux * T;
        g[3] = wm * T + R(0.5) * uy * T;
        g[4] = wm * T - R(0.5) * uy * T;
        g[5] = wm * T + R(0.5) * uz * T;
        g[6] = wm * T - R(0.5) * uz * T;
    }
}

// ------------------------------------------------------------ D2Q9 + D2Q5

// Density deviation, velocity (with the half force) and T of shifted D2Q9
// populations h and D2Q5 populations g.
template <typename R, bool TH>
__device__ __forceinline__ Macro<R> macros(const R (&h)[Q9], const R (&g)[Q5], const Collision<R>& c)
{
    R drho = h[0];
#pragma unroll
    for (int q = 1; q < Q9; ++q) drho += h[q];
    const R jx = (h[1] - h[2]) + (h[5] - h[6]) + (h[7] - h[8]);
    const R jy = (h[3] - h[4]) + (h[5] - h[6]) - (h[7] - h[8]);
    Macro<R> m;
    m.rho = R(1) + drho;
    m.T = R(0);
    R ax = c.accel[0], ay = c.accel[1];
    if (TH) {
        R T = g[0];
#pragma unroll
        for (int k = 1; k < Q5; ++k) T += g[k];
        m.T = T;
        const R dT = T - c.T0;
        ax += c.gbeta[0] * dT;
        ay += c.gbeta[1] * dT;
    }
    const R ir = R(1) / m.rho;
    m.ux = jx * ir + R(0.5) * ax;
    m.uy = jy * ir + R(0.5) * ay;
    m.uz = R(0);
    return m;
}

// One cell's D2Q9 MRT + Guo collision and D2Q5 MRT collision, in place on
// the register arrays.  dm_k = -s_k (m_k - m_eq_k) + (1 - s_k/2) (M F~)_k
// with (M F~) = (0, 6 u.F, -6 u.F, Fx, -Fx, Fy, -Fy, 2(ux Fx - uy Fy),
// ux Fy + uy Fx); the equilibrium moments are rho (1, -2 + 3u^2, 1 - 3u^2,
// ux, -ux, uy, -uy, ux^2 - uy^2, ux uy).  The rest-state weights contribute
// -2 to e and 1 to eps of the shifted moments.
template <typename R, bool TH>
__device__ __forceinline__ void collide(R (&h)[Q9], R (&g)[Q5], const Collision<R>& c)
{
    const R sx = h[1] + h[2], dx = h[1] - h[2];
    const R sy = h[3] + h[4], dy = h[3] - h[4];
    const R a56 = h[5] + h[6], d56 = h[5] - h[6];
    const R a78 = h[7] + h[8], d78 = h[7] - h[8];
    const R Sax = sx + sy, Sdg = a56 + a78;
    const R drho = h[0] + Sax + Sdg;
    const R jx = dx + (d56 + d78);
    const R jy = dy + (d56 - d78);

    const R rho = R(1) + drho;
    R ax = c.accel[0], ay = c.accel[1];
    R T = R(0);
    if (TH) {
        T = (g[0] + g[1]) + (g[2] + g[3]) + g[4];
        const R dT = T - c.T0;
        ax += c.gbeta[0] * dT;
        ay += c.gbeta[1] * dT;
    }
    const R ir = R(1) / rho;
    const R ux = jx * ir + R(0.5) * ax;
    const R uy = jy * ir + R(0.5) * ay;
    const R Fx = rho * ax, Fy = rho * ay;
    const R uxx = ux * ux, uyy = uy * uy;
    const R uu = uxx + uyy;
    const R uF = ux * Fx + uy * Fy;

    const R ne_e = (R(-4) * h[0] - Sax + R(2) * Sdg) + R(2) * drho - R(3) * rho * uu;
    const R ne_eps = (R(4) * h[0] - R(2) * Sax + Sdg) - drho + R(3) * rho * uu;
    const R ne_qx = (R(-2) * dx + (d56 + d78)) + rho * ux;
    const R ne_qy = (R(-2) * dy + (d56 - d78)) + rho * uy;
    const R ne_pxx = (sx - sy) - rho * (uxx - uyy);
    const R ne_pxy = (a56 - a78) - rho * ux * uy;

    const R E = (-c.s2_e * ne_e + (R(1) - R(0.5) * c.s2_e) * (R(6) * uF)) * R(1.0 / 36.0);
    const R P = (-c.s2_eps * ne_eps + (R(1) - R(0.5) * c.s2_eps) * (R(-6) * uF)) * R(1.0 / 36.0);
    const R X = Fx * R(1.0 / 6.0), Y = Fy * R(1.0 / 6.0);
    const R QX = (-c.s2_qx * ne_qx + (R(1) - R(0.5) * c.s2_qx) * (-Fx)) * R(1.0 / 12.0);
    const R QY = (-c.s2_qy * ne_qy + (R(1) - R(0.5) * c.s2_qy) * (-Fy)) * R(1.0 / 12.0);
    const R A = (-c.s2_pxx * ne_pxx + (R(1) - R(0.5) * c.s2_pxx) * (R(2) * (ux * Fx - uy * Fy))) * R(0.25);
    const R B = (-c.s2_pxy * ne_pxy + (R(1) - R(0.5) * c.s2_pxy) * (ux * Fy + uy * Fx)) * R(0.25);

    const R axc = -E - R(2) * P;
    const R dgc = R(2) * E + P;
    const R XQ = X - R(2) * QX, YQ = Y - R(2) * QY;  // axis flux terms
    const R xq = X + QX, yq = Y + QY;                // diagonal flux terms
    h[0] += R(-4) * E + R(4) * P;
    h[1] += axc + A + XQ;
    h[2] += axc + A - XQ;
    h[3] += axc - A + YQ;
    h[4] += axc - A - YQ;
    h[5] += dgc + B + (xq + yq);
    h[6] += dgc + B - (xq + yq);
    h[7] += dgc - B + (xq - yq);
    h[8] += dgc - B - (xq - yq);

    if (TH) {
        const R n1 = g[1] - g[2], n2 = g[3] - g[4];
        const R px = g[1] + g[2], py = g[3] + g[4];
        const R n3 = R(-4) * g[0] + (px + py);
        const R n4 = px - py;
        const R K1 = -c.q2_jx * (n1 - ux * T) * R(0.5);
        const R K2 = -c.q2_jy * (n2 - uy * T) * R(0.5);
        const R K3 = -c.q2_e * (n3 - c.a_T * T) * R(1.0 / 20.0);
        const R K4 = -c.q2_4 * n4 * R(0.25);
        g[0] += R(-4) * K3;
        g[1] += (K3 + K4) + K1;
        g[2] += (K3 + K4) - K1;
        g[3] += (K3 - K4) + K2;
        g[4] += (K3 - K4) - K2;
    }
}

// Shifted D2Q9 equilibrium h_q = f_eq_q - w_q and D2Q5 equilibrium.
template <typename R, bool TH>
__device__ __forceinline__ void equilibrium(R rho, R ux, R uy, R uz, R T, R a_T, R (&h)[Q9], R (&g)[Q5])
{
    (void)uz;
    const R uu = ux * ux + uy * uy;
    const R drho = rho - R(1);
#pragma unroll
    for (int q = 0; q < Q9; ++q) {
        const R cu = R(cx9(q)) * ux + R(cy9(q)) * uy;
        h[q] = R(w9(q)) * (drho + rho * (R(3) * cu + R(4.5) * cu * cu - R(1.5) * uu));
    }
    if (TH) {
        const R wm = (R(4) + a_T) / R(20);
        g[0] = (R(1) - a_T) / R(5) * T;
        g[1] = wm * T + R(0.5) * ux * T;
        g[2] = wm * T - R(0.5) * ux * T;
        g[3] = wm * T + R(0.5) * uy * T;
        g[4] = wm * T - R(0.5) * uy * T;
    }
}

}  // namespace lbm
