// lbm_kernels.hip -- the HIP kernels of the fused lattice Boltzmann step (gfx950).
//
// Every kernel is written once for both lattice pairs of the
// double-distribution model (D3Q19 + D3Q7, and D2Q9 + D2Q5 on one z layer),
// given as a compile-time descriptor L (lbm_lattice.hpp).
//
// Layout: structure of arrays, one plane per population direction, cell
// index x + nx*(y + ny*z) inside a plane ("Multi-GPU thermal lattice
// Boltzmann simulations using OpenACC and MPI", Sec. 3: SoA so that
// neighbouring threads touch neighbouring data), cut into tiles of
// consecutive cells that hold all planes of the tile (the collected SoA of
// "GPU Optimization for High-Quality Kinetic Fluid Simulation", Sec. 4.1)
// where the buffers allow; see pos().  One thread per cell, cells flattened,
// so a 64-lane wavefront reads and writes 64 consecutive elements of each
// plane (256 B in fp32) whatever the box shape.
//
// In-place AA streaming ("GPU lattice Boltzmann: streaming layout and
// performance", OneCAD docs): even steps read population q of cell x at
// (q, x) and write the collided value at (opposite(q), x); odd steps read at
// (opposite(q), x - c_q) and write at (q, x + c_q).  Each cell writes exactly
// the slots it read, so one buffer suffices and cells never race.  Solid cells
// are processed like fluid ones (they hold NaN); no fluid cell ever reads a
// value a solid cell wrote: the bounce-back in the odd step (or, in link-pass
// mode, a link scatter) supplies every population that would come from one.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lbm_internal.hpp"

namespace lbm {

namespace {

constexpr int BLOCK = 256;
constexpr int LBM_GROUPS = 261;  // 6 faces + 255 solid labels

// Run-time direction tables of a flow lattice packed into 64-bit constants:
// 2 bits per direction holding c + 1.
template <class L>
__host__ __device__ constexpr uint64_t pack_dirs(int which)
{
    uint64_t v = 0;
    for (int q = 0; q < L::Q; ++q) {
        const int c = which == 0 ? L::cx(q) : (which == 1 ? L::cy(q) : L::cz(q));
        v |= (uint64_t)(c + 1) << (2 * q);
    }
    return v;
}
template <class L>
struct Packed {
    static constexpr uint64_t X = pack_dirs<L>(0), Y = pack_dirs<L>(1), Z = pack_dirs<L>(2);
};

__device__ __forceinline__ int dir_comp(uint64_t packed, int q) { return (int)((packed >> (2 * q)) & 3u) - 1; }

// Wrapped neighbour offsets of one cell: a cell's coordinates are computed
// once and each axis wraps with a compare and an add.
// On one z layer (DIMS = 2) z is 0 and the z offsets vanish.
template <int DIMS>
struct Nbr {
    int32_t xm, xp, ym, yp, zm, zp;
    uint32_t faces;  // bit f: the cell touches box face f (x-, x+, y-, y+, z-, z+)
    int32_t x, y, z;

    __device__ __forceinline__ Nbr(const Geometry& G, int32_t cell)
    {
        const uint32_t r = divide((uint32_t)cell, G.div_nx);
        x = cell - (int32_t)r * G.nx;
        if (DIMS == 2) {
            z = 0;
            y = (int32_t)r;
        } else {
            z = (int32_t)divide(r, G.div_ny);
            y = (int32_t)r - z * G.ny;
        }
        xm = (x == 0) ? G.nx - 1 : -1;
        xp = (x == G.nx - 1) ? 1 - G.nx : 1;
        ym = (y == 0) ? (G.ny - 1) * G.nx : -G.nx;
        yp = (y == G.ny - 1) ? (1 - G.ny) * G.nx : G.nx;
        zm = DIMS == 2 ? 0 : (((int32_t)z == 0) ? (G.nz - 1) * G.nxy : -G.nxy);
        zp = DIMS == 2 ? 0 : (((int32_t)z == G.nz - 1) ? (1 - G.nz) * G.nxy : G.nxy);
        faces = (x == 0 ? 1u : 0u) | (x == G.nx - 1 ? 2u : 0u) | (y == 0 ? 4u : 0u) | (y == G.ny - 1 ? 8u : 0u) |
                ((int32_t)z == 0 ? 16u : 0u) | ((int32_t)z == G.nz - 1 ? 32u : 0u);
    }
    // offset of the cell at x + (cx, cy, cz), each component in {-1, 0, 1}
    __device__ __forceinline__ int32_t at(int cx, int cy, int cz) const
    {
        return (cx > 0 ? xp : (cx < 0 ? xm : 0)) + (cy > 0 ? yp : (cy < 0 ? ym : 0)) +
               (cz > 0 ? zp : (cz < 0 ? zm : 0));
    }
};

// Position of population q of cell idx in a population buffer.  Cells are
// grouped in tiles of 2^tile_lg consecutive cells; a tile holds the buffer's
// planes one after another (plane q at q * qstride inside the tile) and
// consecutive tiles lie ts elements apart.  With tile_lg = 31 the whole box
// is one tile: plain structure of arrays, planes qstride apart.  The plane
// part q * qstride is uniform across the wavefront (a scalar base) and the
// per-lane part, the same for every plane, is a 32-bit element offset (the
// host keeps every buffer below 2^32 elements), scaled to bytes in 64-bit
// arithmetic so that tiled buffers may reach 16 GiB (fp32) or 32 GiB (fp64).
// Each access thus takes a 64-bit address per lane; where a cell loads and
// stores the same slot (the odd step: population opp(q) comes from, and q
// goes to, (q, x + c_q)) one address serves both.  On MI355X this measured
// as fast as the scalar-base + 32-bit-byte-offset form on the boxes that fit
// the latter (256^3: within 0.2 %), and forcing the scalar-base form on both
// accesses of a shared slot made the odd step 6 % slower.
struct Slot {
    int64_t plane;  // uniform: element offset of the plane's base
    uint32_t off;   // per lane: element offset from the plane's base
};

__device__ __forceinline__ Slot pos(const Geometry& G, uint32_t ts, int q, int32_t idx)
{
    const uint32_t u = (uint32_t)idx;
    return Slot{(int64_t)q * G.qstride, __umul24(u >> G.tile_lg, ts) + (u & G.tile_mask)};
}
// flow-lattice (f) and temperature-lattice (g) buffers
__device__ __forceinline__ Slot posf(const Geometry& G, int q, int32_t idx) { return pos(G, G.tile_f, q, idx); }
__device__ __forceinline__ Slot posg(const Geometry& G, int q, int32_t idx) { return pos(G, G.tile_g, q, idx); }
__device__ __forceinline__ Slot posb(const Geometry& G, bool temp, int q, int32_t idx)
{
    return temp ? posg(G, q, idx) : posf(G, q, idx);
}

template <typename R>
__device__ __forceinline__ R ld(const R* base, Slot p)
{
    const char* plane = reinterpret_cast<const char*>(base + p.plane);
    return *reinterpret_cast<const R*>(plane + (uint64_t)p.off * sizeof(R));
}
template <typename R>
__device__ __forceinline__ void st(R* base, Slot p, R v)
{
    char* plane = reinterpret_cast<char*>(base + p.plane);
    *reinterpret_cast<R*>(plane + (uint64_t)p.off * sizeof(R)) = v;
}

// ------------------------------------------------------ boundaries

// Flow-lattice directions leaving the box through face f (x-, x+, y-, y+, z-, z+).
template <class L>
__host__ __device__ constexpr uint32_t dirs_through(int f)
{
    uint32_t m = 0;
    for (int q = 1; q < L::Q; ++q) {
        const int c = (f >> 1) == 0 ? L::cx(q) : ((f >> 1) == 1 ? L::cy(q) : L::cz(q));
        if ((f & 1) ? c > 0 : c < 0) m |= 1u << q;
    }
    return m;
}

// Face crossed by temperature-lattice direction k (1..6, or 1..4 in 2D).
__host__ __device__ constexpr int face7(int k) { return (k - 1) ^ 1; }

// Blocked directions of one cell for the in-kernel bounce-back: `wall` holds
// the directions that leave through a no-slip face (from the coordinates),
// `solid` those whose neighbour is a solid cell (mask of a fluid cell), and
// `claim` on a solid cell the directions whose odd-step slot a fluid
// neighbour re-reads and re-stores (mask bits of a solid cell).
struct Blocked {
    uint32_t wall, solid, claim;
    bool is_solid;
};

template <class L, typename R>
__device__ __forceinline__ Blocked blocked_dirs(const Bounce<R>& bb, const uint32_t* mask, int32_t cell,
                                                uint32_t faces)
{
    Blocked b;
    const uint32_t fw = faces & (uint32_t)bb.walls;
    b.wall = ((fw & 1u) ? dirs_through<L>(0) : 0u) | ((fw & 2u) ? dirs_through<L>(1) : 0u) |
             ((fw & 4u) ? dirs_through<L>(2) : 0u) | ((fw & 8u) ? dirs_through<L>(3) : 0u) |
             ((fw & 16u) ? dirs_through<L>(4) : 0u) | ((fw & 32u) ? dirs_through<L>(5) : 0u);
    uint32_t m = 0u;
    if (mask && ((mask[bb.near_off + (cell >> 5)] >> (cell & 31)) & 1u)) m = mask[cell];
    b.is_solid = (m & MASK_SOLID) != 0;
    b.solid = b.is_solid ? 0u : m;
    b.claim = b.is_solid ? (m & ~MASK_SOLID) : 0u;
    return b;
}

// The value a temperature population takes when it bounces in direction k's face or
// off a solid: anti-bounce-back gw - g (Dirichlet) or g (adiabatic).
template <typename R>
__device__ __forceinline__ R bounce7(const Bounce<R>& bb, const Blocked& b, int k, R v)
{
    if ((b.wall >> k) & 1u) {
        const int f = face7(k);
        return ((bb.face_dirichlet >> f) & 1) ? bb.face_gw[f] - v : v;
    }
    return bb.solid_dirichlet ? bb.solid_gw - v : v;
}

// Reflection of flow direction p across a face of axis a: the a component
// of c_p reversed.
template <class L>
__host__ __device__ constexpr int refl(int a, int p)
{
    for (int r = 0; r < L::Q; ++r)
        if (L::cx(r) == (a == 0 ? -L::cx(p) : L::cx(p)) && L::cy(r) == (a == 1 ? -L::cy(p) : L::cy(p)) &&
            L::cz(r) == (a == 2 ? -L::cz(p) : L::cz(p)))
            return r;
    return 0;
}

// The directions of one cell that leave the box, by the axis of the face
// that governs them (the first crossed axis in x, y, z order) and by that
// face's rule.  SLIP keeps only directions that cross a single face: one
// that crosses two faces bounces back like a wall link.
struct FaceRules {
    uint32_t ax, ay, az;
    uint32_t slip, vel, pres;
};

template <class L, typename R>
__device__ __forceinline__ FaceRules face_rules(const Bounce<R>& bb, uint32_t faces)
{
    const uint32_t fw = faces & (uint32_t)bb.walls;
    const uint32_t cx = ((fw & 1u) ? dirs_through<L>(0) : 0u) | ((fw & 2u) ? dirs_through<L>(1) : 0u);
    const uint32_t cy = ((fw & 4u) ? dirs_through<L>(2) : 0u) | ((fw & 8u) ? dirs_through<L>(3) : 0u);
    const uint32_t cz = ((fw & 16u) ? dirs_through<L>(4) : 0u) | ((fw & 32u) ? dirs_through<L>(5) : 0u);
    FaceRules r;
    r.ax = cx;
    r.ay = cy & ~cx;
    r.az = cz & ~(cx | cy);
    uint32_t sl = 0u, ve = 0u, pr = 0u;
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const uint32_t gov = (f < 2 ? r.ax : (f < 4 ? r.ay : r.az)) & dirs_through<L>(f);
        if ((bb.slip >> f) & 1) sl |= gov;
        if ((bb.vel >> f) & 1) ve |= gov;
        if ((bb.pres >> f) & 1) pr |= gov;
    }
    r.slip = sl & ~((cx & (cy | cz)) | (cy & cz));
    r.vel = ve;
    r.pres = pr;
    return r;
}

// Axis and face that govern a leaving direction p.
__device__ __forceinline__ int gov_axis(const FaceRules& r, int p)
{
    return ((r.ax >> p) & 1u) ? 0 : (((r.ay >> p) & 1u) ? 1 : 2);
}
template <class L>
__device__ __forceinline__ int gov_face(const FaceRules& r, int p)
{
    const int a = gov_axis(r, p);
    const int c = a == 0 ? L::cx(p) : (a == 1 ? L::cy(p) : L::cz(p));
    return 2 * a + (c > 0 ? 1 : 0);
}

// VELOCITY link (Ladd's moving wall): the returning population is
// f_p^+ - 6 w_p rho_w c_p.u_w; this is the subtracted term.
template <class L, typename R>
__device__ __forceinline__ R vel_shift(const Bounce<R>& bb, int f, int p)
{
    const R cu = (R)L::cx(p) * bb.face_u[f][0] + (R)L::cy(p) * bb.face_u[f][1] + (R)L::cz(p) * bb.face_u[f][2];
    return (R)(6.0 * L::w(p)) * bb.face_rho[f] * cu;
}

// PRESSURE link (anti-bounce-back at the wall density): the returning
// population f = -f_p^+ + 2 w_p rho_w [1 + 9/2 (c_p.u)^2 - 3/2 u.u], written
// for shifted storage (f = h + w_p).
template <class L, typename R>
__device__ __forceinline__ R pres_value(const Bounce<R>& bb, int f, int p, R hout, R ux, R uy, R uz)
{
    const R cu = (R)L::cx(p) * ux + (R)L::cy(p) * uy + (R)L::cz(p) * uz;
    const R uu = ux * ux + uy * uy + uz * uz;
    return (R)(2.0 * L::w(p)) * (bb.face_rho[f] * (R(1) + R(4.5) * cu * cu - R(1.5) * uu) - R(1)) - hout;
}

// A cell's slot in the velocity planes of PRESSURE face f.
template <typename R, int D>
__device__ __forceinline__ int64_t face_slot(const Bounce<R>& bb, const Geometry& G, int f, const Nbr<D>& nb)
{
    const int32_t i = f < 2 ? nb.y + G.ny * nb.z : (f < 4 ? nb.x + G.nx * nb.z : nb.x + G.nx * nb.y);
    return bb.face_off[f] + i;
}

// Keep a cell's velocity for each PRESSURE face it lies on (read by the
// two-buffer pull and by the force pass).
template <typename R, int D>
__device__ __forceinline__ void keep_face_velocity(const Bounce<R>& bb, const Geometry& G, const Nbr<D>& nb, R ux,
                                                   R uy, R uz)
{
    const uint32_t fp = nb.faces & (uint32_t)bb.pres;
#pragma unroll
    for (int f = 0; f < 6; ++f)
        if ((fp >> f) & 1u) {
            const int64_t i = face_slot(bb, G, f, nb);
            bb.face_vel[i] = ux;
            bb.face_vel[i + bb.face_area[f]] = uy;
            bb.face_vel[i + 2 * bb.face_area[f]] = uz;
        }
}

// In place, population q of fluid cell x after an odd step's streaming when
// the link (x, opp q) is blocked: read where the preceding even step left
// the returning population.  Wall, solid and PRESSURE links: the cell's own
// slot (q, x) (an even step stores PRESSURE links already anti-bounced);
// VELOCITY: the same, less the moving-wall term; SLIP: the population sent
// from x - c_t along q reflected, at (opposite(q reflected), x - c_t).
template <class L, typename R, int BND>
__device__ __forceinline__ R blocked_inflow(const R* f, const Geometry& G, int32_t cell, const Nbr<L::DIMS>& nb,
                                            const FaceRules& fr, const Bounce<R>& bb, int q)
{
    const int p = opp(q);
    if (BND == 2 && ((fr.slip >> p) & 1u)) {
        const int a = gov_axis(fr, p);
        const int src = a == 0 ? refl<L>(0, q) : (a == 1 ? refl<L>(1, q) : refl<L>(2, q));
        const int32_t y = cell + nb.at(a == 0 ? 0 : -L::cx(q), a == 1 ? 0 : -L::cy(q), a == 2 ? 0 : -L::cz(q));
        return ld(f, posf(G, opp(src), y));
    }
    R v = ld(f, posf(G, q, cell));
    if (BND == 2 && ((fr.vel >> p) & 1u)) v -= vel_shift<L>(bb, gov_face<L>(fr, p), p);
    return v;
}

// In place, an odd step's blocked outflow p of fluid cell x, stored where the
// next (even) step reads the returning population: (opposite(p), x) with the
// link's rule applied, or for SLIP (p reflected, x + c_t).
template <class L, typename R, int BND>
__device__ __forceinline__ void blocked_outflow(R* f, const Geometry& G, int32_t cell, const Nbr<L::DIMS>& nb,
                                                const FaceRules& fr, const Bounce<R>& bb, int p, R h, R ux, R uy,
                                                R uz)
{
    if (BND == 2 && ((fr.slip >> p) & 1u)) {
        const int a = gov_axis(fr, p);
        const int dst = a == 0 ? refl<L>(0, p) : (a == 1 ? refl<L>(1, p) : refl<L>(2, p));
        st(f, posf(G, dst, cell + nb.at(a == 0 ? 0 : L::cx(p), a == 1 ? 0 : L::cy(p), a == 2 ? 0 : L::cz(p))),
           h);
        return;
    }
    R v = h;
    if (BND == 2 && ((fr.vel >> p) & 1u)) v = h - vel_shift<L>(bb, gov_face<L>(fr, p), p);
    if (BND == 2 && ((fr.pres >> p) & 1u)) v = pres_value<L>(bb, gov_face<L>(fr, p), p, h, ux, uy, uz);
    st(f, posf(G, opp(p), cell), v);
}

// ------------------------------------------------------------ AA step


// One fused time step in place.  With BND the step also applies the
// half-way boundary rules at non-periodic faces and solid cells
// ("Multi-GPU thermal lattice Boltzmann simulations using OpenACC and MPI",
// Sec. 2); without it the box streams as if periodic and link passes fix
// the blocked directions.  BND = 1: no-slip walls and solids only; BND = 2:
// also SLIP, VELOCITY and PRESSURE faces.
// All bounce-back work happens in the odd step; the even step is the plain
// kernel for every cell (solid cells compute on NaN in their own slots),
// except that cells on a PRESSURE face store their leaving populations
// already anti-bounced (the rule needs the cell's velocity of that step):
//  * even step: every cell stores f_p^+ at (opp p, x);
//  * odd step, inflow: a population q whose upstream cell x - c_q is across
//    a face or solid is the returning f_opp(q)^+(x) from the even step, which
//    sits in (q, x) of the cell itself -- it is read there (blocked_inflow);
//  * odd step, outflow: f_p^+ for a blocked direction p is stored at
//    (opp p, x), where the next (even) step reads it (blocked_outflow).  Its
//    usual slot is skipped when p leaves through a face (the addressing
//    wraps onto the cell across the box, whose slot that is) and kept when p
//    points at a solid cell (only that solid cell reads it next).
// A solid cell skips its odd-step stores into slots a fluid neighbour claims
// this way (mask bits) and into wrapped slots across a face.  No slot is
// touched by two cells in one step.
template <class L, typename R, bool TH, int BND>
__global__ void __launch_bounds__(BLOCK) k_aa_step(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    R* __restrict__ f = a.f;
    R* __restrict__ gg = a.g;
    R h[L::Q];
    R g[L::QT];
    if (a.parity == 0) {
#pragma unroll
        for (int q = 0; q < L::Q; ++q) h[q] = ld(f, posf(G, q, cell));
        if (TH) {
#pragma unroll
            for (int k = 0; k < L::QT; ++k) g[k] = ld(gg, posg(G, k, cell));
        }
        uint32_t pdirs = 0u;
        FaceRules fr{};
        R ux = R(0), uy = R(0), uz = R(0);
        if (BND == 2 && a.bb.pres) {
            const Nbr<L::DIMS> nb(G, cell);
            if ((nb.faces & (uint32_t)a.bb.pres) && !(a.mask && (a.mask[cell] & MASK_SOLID))) {
                fr = face_rules<L>(a.bb, nb.faces);
                pdirs = fr.pres;
                const Macro<R> m = macros<R, TH>(h, g, a.col);
                ux = m.ux;
                uy = m.uy;
                uz = m.uz;
                keep_face_velocity(a.bb, G, nb, ux, uy, uz);
            }
        }
        collide<R, TH>(h, g, a.col);
        if (BND == 2 && pdirs) {
#pragma unroll
            for (int p = 1; p < L::Q; ++p)
                if ((pdirs >> p) & 1u) h[p] = pres_value<L>(a.bb, gov_face<L>(fr, p), p, h[p], ux, uy, uz);
        }
#pragma unroll
        for (int q = 0; q < L::Q; ++q) st(f, posf(G, opp(q), cell), h[q]);
        if (TH) {
#pragma unroll
            for (int k = 0; k < L::QT; ++k) st(gg, posg(G, opp(k), cell), g[k]);
        }
        return;
    }
    const Nbr<L::DIMS> nb(G, cell);
    Blocked b{0u, 0u, 0u, false};
    if (BND) b = blocked_dirs<L>(a.bb, a.mask, cell, nb.faces);
    const uint32_t blk = b.wall | b.solid;           // a fluid cell's blocked directions
    const uint32_t skip = b.wall | b.claim;          // usual odd-step stores to leave out
    const bool near = BND && !b.is_solid && blk != 0;
    FaceRules fr{};
    if (BND == 2 && near) fr = face_rules<L>(a.bb, nb.faces);
#pragma unroll
    for (int q = 0; q < L::Q; ++q) h[q] = ld(f, posf(G, opp(q), cell + nb.at(-L::cx(q), -L::cy(q), -L::cz(q))));
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k)
            g[k] = ld(gg, posg(G, opp(k), cell + nb.at(-L::cxT(k), -L::cyT(k), -L::czT(k))));
    }
    if (near) {
#pragma unroll
        for (int q = 1; q < L::Q; ++q)
            if ((blk >> opp(q)) & 1u) h[q] = blocked_inflow<L, R, BND>(f, G, cell, nb, fr, a.bb, q);
        if (TH) {
#pragma unroll
            for (int k = 1; k < L::QT; ++k)
                if ((blk >> opp(k)) & 1u) g[k] = bounce7(a.bb, b, opp(k), ld(gg, posg(G, k, cell)));
        }
    }
    R ux = R(0), uy = R(0), uz = R(0);
    if (BND == 2 && fr.pres) {
        const Macro<R> m = macros<R, TH>(h, g, a.col);
        ux = m.ux;
        uy = m.uy;
        uz = m.uz;
        keep_face_velocity(a.bb, G, nb, ux, uy, uz);
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < L::Q; ++q)
        if (!BND || !((skip >> q) & 1u)) st(f, posf(G, q, cell + nb.at(L::cx(q), L::cy(q), L::cz(q))), h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k)
            if (!BND || !((skip >> k) & 1u))
                st(gg, posg(G, k, cell + nb.at(L::cxT(k), L::cyT(k), L::czT(k))), g[k]);
    }
    if (near) {
#pragma unroll
        for (int p = 1; p < L::Q; ++p)
            if ((blk >> p) & 1u) blocked_outflow<L, R, BND>(f, G, cell, nb, fr, a.bb, p, h[p], ux, uy, uz);
        if (TH) {
#pragma unroll
            for (int k = 1; k < L::QT; ++k)
                if ((blk >> k) & 1u) st(gg, posg(G, opp(k), cell), bounce7(a.bb, b, k, g[k]));
        }
    }
}

// ------------------------------------------------- two buffers (A-B)

// Collide in place: every population stays in its own slot (solid cells
// compute on NaN in theirs; no fluid cell pulls from a solid slot).  Cells on
// a PRESSURE face keep their velocity for the pull's anti-bounce-back.
template <class L, typename R, bool TH, int BND>
__global__ void __launch_bounds__(BLOCK) k_ab_collide(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    R h[L::Q];
    R g[L::QT];
#pragma unroll
    for (int q = 0; q < L::Q; ++q) h[q] = ld(a.f, posf(G, q, cell));
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k) g[k] = ld(a.g, posg(G, k, cell));
    }
    if (BND == 2 && a.bb.pres) {
        const Nbr<L::DIMS> nb(G, cell);
        if ((nb.faces & (uint32_t)a.bb.pres) && !(a.mask && (a.mask[cell] & MASK_SOLID))) {
            const Macro<R> m = macros<R, TH>(h, g, a.col);
            keep_face_velocity(a.bb, G, nb, m.ux, m.uy, m.uz);
        }
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < L::Q; ++q) st(a.f, posf(G, q, cell), h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k) st(a.g, posg(G, k, cell), g[k]);
    }
}

// Pull into the other buffer: B(q, x) = A(q, x - c_q).  With BND, when
// x - c_q is across a face or a solid cell the population returns by the
// link's rule: from x itself, B(q, x) = A(opp q, x) (bounce-back; less the
// moving-wall term for VELOCITY; anti-bounce-back for PRESSURE, and for a
// Dirichlet temperature link), or for SLIP from x - c_t along q reflected.
template <class L, typename R, bool TH, int BND>
__global__ void __launch_bounds__(BLOCK) k_ab_pull(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const Nbr<L::DIMS> nb(G, cell);
    Blocked b{0u, 0u, 0u, false};
    if (BND) b = blocked_dirs<L>(a.bb, a.mask, cell, nb.faces);
    const uint32_t blk = b.is_solid ? 0u : (b.wall | b.solid);
    FaceRules fr{};
    if (BND == 2 && blk) fr = face_rules<L>(a.bb, nb.faces);
    R ux = R(0), uy = R(0), uz = R(0);
    if (BND == 2 && fr.pres) {
        const int f = __builtin_ctz(nb.faces & (uint32_t)a.bb.pres);  // any of its PRESSURE faces
        const int64_t i = face_slot(a.bb, G, f, nb);
        ux = a.bb.face_vel[i];
        uy = a.bb.face_vel[i + a.bb.face_area[f]];
        uz = a.bb.face_vel[i + 2 * a.bb.face_area[f]];
    }
#pragma unroll
    for (int q = 0; q < L::Q; ++q) {
        R v = ld(a.f, posf(G, q, cell + nb.at(-L::cx(q), -L::cy(q), -L::cz(q))));
        const int p = opp(q);
        if (BND && ((blk >> p) & 1u)) {
            if (BND == 2 && ((fr.slip >> p) & 1u)) {
                const int ax = gov_axis(fr, p);
                const int src = ax == 0 ? refl<L>(0, q) : (ax == 1 ? refl<L>(1, q) : refl<L>(2, q));
                v = ld(a.f, posf(G, src,
                                cell + nb.at(ax == 0 ? 0 : -L::cx(q), ax == 1 ? 0 : -L::cy(q), ax == 2 ? 0 : -L::cz(q))));
            } else {
                v = ld(a.f, posf(G, p, cell));
                if (BND == 2 && ((fr.vel >> p) & 1u)) v -= vel_shift<L>(a.bb, gov_face<L>(fr, p), p);
                if (BND == 2 && ((fr.pres >> p) & 1u)) v = pres_value<L>(a.bb, gov_face<L>(fr, p), p, v, ux, uy, uz);
            }
        }
        st(a.f2, posf(G, q, cell), v);
    }
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k) {
            R v = ld(a.g, posg(G, k, cell + nb.at(-L::cxT(k), -L::cyT(k), -L::czT(k))));
            if (BND && ((blk >> opp(k)) & 1u)) v = bounce7(a.bb, b, opp(k), ld(a.g, posg(G, opp(k), cell)));
            st(a.g2, posg(G, k, cell), v);
        }
    }
}

// Two buffers in one pass: every cell loads its populations from A where
// they sit at time t (its own slots), collides, and pushes f_q^+ to
// B(q, x + c_q).  A blocked direction (a face or a solid cell at x + c_q) is
// stored by the link's rule where the cell itself reads it next, exactly as
// the in-place odd step stores it (blocked_outflow); a solid cell leaves out
// the slots that a fluid neighbour fills that way (its mask bits), and no
// cell stores across a no-slip face.  B then holds every population at time
// t + 1 in its own slot, as after a pull.
template <class L, typename R, bool TH, int BND>
__global__ void __launch_bounds__(BLOCK) k_ab_push(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    R* __restrict__ fb = a.f2;
    R* __restrict__ gb = a.g2;
    R h[L::Q];
    R g[L::QT];
#pragma unroll
    for (int q = 0; q < L::Q; ++q) h[q] = ld(a.f, posf(G, q, cell));
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k) g[k] = ld(a.g, posg(G, k, cell));
    }
    const Nbr<L::DIMS> nb(G, cell);
    Blocked b{0u, 0u, 0u, false};
    if (BND) b = blocked_dirs<L>(a.bb, a.mask, cell, nb.faces);
    const uint32_t blk = b.wall | b.solid;           // a fluid cell's blocked directions
    const uint32_t skip = b.wall | b.claim;          // usual stores to leave out
    const bool near = BND && !b.is_solid && blk != 0;
    FaceRules fr{};
    if (BND == 2 && near) fr = face_rules<L>(a.bb, nb.faces);
    R ux = R(0), uy = R(0), uz = R(0);
    if (BND == 2 && fr.pres) {
        const Macro<R> m = macros<R, TH>(h, g, a.col);
        ux = m.ux;
        uy = m.uy;
        uz = m.uz;
        keep_face_velocity(a.bb, G, nb, ux, uy, uz);
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < L::Q; ++q)
        if (!BND || !((skip >> q) & 1u)) st(fb, posf(G, q, cell + nb.at(L::cx(q), L::cy(q), L::cz(q))), h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k)
            if (!BND || !((skip >> k) & 1u))
                st(gb, posg(G, k, cell + nb.at(L::cxT(k), L::cyT(k), L::czT(k))), g[k]);
    }
    if (near) {
#pragma unroll
        for (int p = 1; p < L::Q; ++p)
            if ((blk >> p) & 1u) blocked_outflow<L, R, BND>(fb, G, cell, nb, fr, a.bb, p, h[p], ux, uy, uz);
        if (TH) {
#pragma unroll
            for (int k = 1; k < L::QT; ++k)
                if ((blk >> k) & 1u) st(gb, posg(G, opp(k), cell), bounce7(a.bb, b, k, g[k]));
        }
    }
}

// ------------------------------------------------------------ links

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// The slots one link reads and writes.  p is the direction from the fluid
// cell x towards the wall or solid; the population sent along p comes back
// along opp(p).  In place, after an even step the collided f_p(x) sits in
// (opp p, x) and must land where the next (odd) step reads f_opp(p)(x), which
// is (p, x + c_p); after an odd step it sits in (p, x + c_p) and must land in
// (opp p, x), which the next (even) step reads.  Two buffers: the collided
// value is A(p, x) and the streamed one B(opp p, x).
struct LinkSlots {
    int32_t src_plane, src_idx, dst_plane, dst_idx;
};

__device__ __forceinline__ LinkSlots link_slots(int mode, int p, int32_t cell, int32_t cellw)
{
    LinkSlots s;
    if (mode == LINK_AA_AFTER_EVEN) {
        s.src_plane = opp(p);
        s.src_idx = cell;
        s.dst_plane = p;
        s.dst_idx = cellw;
    } else if (mode == LINK_AA_AFTER_ODD) {
        s.src_plane = p;
        s.src_idx = cellw;
        s.dst_plane = opp(p);
        s.dst_idx = cell;
    } else {
        s.src_plane = p;
        s.src_idx = cell;
        s.dst_plane = opp(p);
        s.dst_idx = cell;
    }
    return s;
}

// Per-link contribution to the group sums.  A flow-lattice link hands the boundary
// the momentum it carries out minus what it brings back, c_p f_out - c_in
// f_in (stored values are f - w): 2 c_p f_p^+ for a wall or solid,
// (c_p - c_p reflected) f_p^+ for SLIP, c_p (f_out + f_in) for VELOCITY and
// PRESSURE.  A Dirichlet temperature link passes w T_w - 2 g_p^+ into the fluid.
// `returned` says whether v is the returning value (else the leaving one);
// a PRESSURE link needs only the cell's velocity, from the face planes.
struct LinkSum {
    double fx, fy, fz, q;
};

template <class L>
__device__ __forceinline__ int refl_rt(int a, int p)
{
    const int c[3] = {dir_comp(Packed<L>::X, p), dir_comp(Packed<L>::Y, p), dir_comp(Packed<L>::Z, p)};
    for (int r = 1; r < L::Q; ++r)
        if (dir_comp(Packed<L>::X, r) == (a == 0 ? -c[0] : c[0]) && dir_comp(Packed<L>::Y, r) == (a == 1 ? -c[1] : c[1]) &&
            dir_comp(Packed<L>::Z, r) == (a == 2 ? -c[2] : c[2]))
            return r;
    return 0;
}

template <class L, typename R>
__device__ __forceinline__ LinkSum link_sum(const LinkArgs<R>& a, uint32_t meta, int p, int32_t grp, R v,
                                            bool returned, int64_t l)
{
    LinkSum c{0.0, 0.0, 0.0, 0.0};
    if (meta & LINK_TEMP) {
        if (meta & LINK_DIRICHLET) c.q = a.omega * a.wall_T[grp] - 2.0 * (double)v;
        return c;
    }
    const double cp[3] = {(double)dir_comp(Packed<L>::X, p), (double)dir_comp(Packed<L>::Y, p), (double)dir_comp(Packed<L>::Z, p)};
    const double w = L::w(p);
    const uint32_t rule = (meta >> LINK_RULE_SHIFT) & 3u;
    double s = 0.0;  // F = s c_p, except SLIP
    if (rule == RULE_WALL) {
        s = 2.0 * ((double)v + w);
    } else if (rule == RULE_SLIP) {
        const int ax = (int)((meta >> LINK_AXIS_SHIFT) & 3u);
        const double fv = 2.0 * cp[ax] * ((double)v + w);
        c.fx = ax == 0 ? fv : 0.0;
        c.fy = ax == 1 ? fv : 0.0;
        c.fz = ax == 2 ? fv : 0.0;
        return c;
    } else if (rule == RULE_VELOCITY) {
        const double cu = cp[0] * (double)a.bb.face_u[grp][0] + cp[1] * (double)a.bb.face_u[grp][1] +
                          cp[2] * (double)a.bb.face_u[grp][2];
        const double shift = 6.0 * w * (double)a.bb.face_rho[grp] * cu;
        const double hout = returned ? (double)v + shift : (double)v;
        s = 2.0 * (hout + w) - shift;
    } else {
        const int64_t i = a.bb.face_off[grp] + a.cellw[l];
        const double ux = (double)a.bb.face_vel[i], uy = (double)a.bb.face_vel[i + a.bb.face_area[grp]],
                     uz = (double)a.bb.face_vel[i + 2 * a.bb.face_area[grp]];
        const double cu = cp[0] * ux + cp[1] * uy + cp[2] * uz;
        s = 2.0 * w * (double)a.bb.face_rho[grp] * (1.0 + 4.5 * cu * cu - 1.5 * (ux * ux + uy * uy + uz * uz));
    }
    c.fx = cp[0] * s;
    c.fy = cp[1] * s;
    c.fz = cp[2] * s;
    return c;
}

// Value a link writes: bounce-back f_pbar = f_p^+ (no-slip), anti-bounce-back
// g_pbar = -g_p^+ + w T_w (Dirichlet T), bounce-back g_pbar = g_p^+ (adiabatic).
template <typename R>
__device__ __forceinline__ R link_value(const LinkArgs<R>& a, uint32_t meta, int32_t grp, R v)
{
    if ((meta & LINK_TEMP) && (meta & LINK_DIRICHLET)) return (R)(a.omega * a.wall_T[grp]) - v;
    return v;
}

// Gather (wall links): read every link's post-collision source into scratch
// before any link writes.  A wall link's destination wraps through the
// periodic addressing onto the source of its partner link on the opposite
// face, so the two passes keep every source intact.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_gather(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const uint32_t meta = a.meta[l];
    const bool t7 = (meta & LINK_TEMP) != 0;
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    const R* src = t7 ? a.g_src : a.f_src;
    a.scratch[l] = ld(src, posb(a.geo, t7, sl.src_plane, sl.src_idx));
}

// Scatter (wall links): write each gathered value where the next step reads it.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_scatter(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const uint32_t meta = a.meta[l];
    const bool t7 = (meta & LINK_TEMP) != 0;
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    R* dst = t7 ? a.g_dst : a.f_dst;
    st(dst, posb(a.geo, t7, sl.dst_plane, sl.dst_idx), link_value(a, meta, grp, a.scratch[l]));
}

// Direct pass (wall links with two buffers): sources lie in one buffer and
// destinations in the other, so gather and scatter merge into one pass.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_direct(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const uint32_t meta = a.meta[l];
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    const bool g7 = (meta & LINK_TEMP) != 0;
    const R v = ld(g7 ? a.g_src : a.f_src, posb(a.geo, g7, sl.src_plane, sl.src_idx));
    st(g7 ? a.g_dst : a.f_dst, posb(a.geo, g7, sl.dst_plane, sl.dst_idx), link_value(a, meta, grp, v));
}

// Force pass, on a submission's last step only, over every link.  It reads
// the bounced population f_p^+ of each link where the step left it: with
// in-kernel bounce-back (opp p, x) in place (the even step's usual store or
// the odd step's bounce-back store); with link passes the scatter
// destination; with two buffers B(opp p, x).  Values a Dirichlet temperature
// link stores after anti-bounce-back are converted back.  Per link: the
// momentum exchange 2 c_p f_p^+ and the heat w T_w - 2 g_p^+ (link_sum).
template <class L, typename R>
__device__ __forceinline__ LinkSum link_force_term(const LinkArgs<R>& a, int64_t l)
{
    const uint32_t meta = a.meta[l];
    const int p = (int)(meta & LINK_DIR_MASK);
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const bool g7 = (meta & LINK_TEMP) != 0;
    int32_t plane, idx;
    bool transformed;
    if (a.in_kernel && a.mode != LINK_AB) {
        // even step: the usual store; odd step: the bounce-back store
        plane = opp(p);
        idx = a.cell[l];
        transformed = a.mode == LINK_AA_AFTER_ODD;
    } else {
        // link passes, or the two-buffer pull: the link's destination
        const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
        plane = sl.dst_plane;
        idx = sl.dst_idx;
        transformed = true;
    }
    if (!g7 && transformed && ((meta >> LINK_RULE_SHIFT) & 3u) == RULE_SLIP) {
        // the reflected population landed at x + c_t
        plane = refl_rt<L>((int)((meta >> LINK_AXIS_SHIFT) & 3u), p);
        idx = a.cellw[l];
    }
    R v = ld(g7 ? a.g_dst : a.f_dst, posb(a.geo, g7, plane, idx));
    if (transformed && g7 && (meta & LINK_DIRICHLET)) v = (R)(a.omega * a.wall_T[grp]) - v;
    return link_sum<L>(a, meta, p, grp, v, transformed, l);
}

// The sums are taken in a fixed order, so the same populations give the same
// forces bit for bit: one wavefront per segment (a run of at most
// LINK_SEGMENT links of one group), each lane adding its links in index
// order, then a butterfly over the lanes; k_force_groups then adds each
// group's segments in order.  No atomics.
template <class L, typename R>
__global__ void __launch_bounds__(BLOCK) k_link_force(LinkArgs<R> a)
{
    const int64_t seg = (int64_t)blockIdx.x * (BLOCK / 64) + (threadIdx.x >> 6);
    if (seg >= a.n_seg) return;  // whole wavefronts leave together
    const int64_t end = a.seg_begin[seg + 1];
    LinkSum c{0.0, 0.0, 0.0, 0.0};
    for (int64_t l = a.seg_begin[seg] + (threadIdx.x & 63); l < end; l += 64) {
        const LinkSum t = link_force_term<L>(a, l);
        c.fx += t.fx;
        c.fy += t.fy;
        c.fz += t.fz;
        c.q += t.q;
    }
    c.fx = wave_sum(c.fx);
    c.fy = wave_sum(c.fy);
    c.fz = wave_sum(c.fz);
    c.q = wave_sum(c.q);
    if ((threadIdx.x & 63) == 0) {
        double* out = a.seg_sum + 4 * seg;
        out[0] = c.fx;
        out[1] = c.fy;
        out[2] = c.fz;
        out[3] = c.q;
    }
}

// Per group (one block each): the sum of its segments, thread t adding
// segments t, t + BLOCK, ... in order, then a fixed halving tree over the
// threads in local data share; written to the group's four accumulators (zero
// for a group without links).
__global__ void __launch_bounds__(BLOCK) k_force_groups(const int32_t* group_seg, const double* seg_sum, double* accum)
{
    __shared__ double part[4][BLOCK];
    const int g = (int)blockIdx.x;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int32_t k = group_seg[g] + (int32_t)threadIdx.x; k < group_seg[g + 1]; k += BLOCK) {
        const double* v = seg_sum + 4 * (int64_t)k;
        s0 += v[0];
        s1 += v[1];
        s2 += v[2];
        s3 += v[3];
    }
    part[0][threadIdx.x] = s0;
    part[1][threadIdx.x] = s1;
    part[2][threadIdx.x] = s2;
    part[3][threadIdx.x] = s3;
    __syncthreads();
    for (int h = BLOCK / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
#pragma unroll
            for (int c = 0; c < 4; ++c) part[c][threadIdx.x] += part[c][threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x < 4) accum[4 * g + threadIdx.x] = part[threadIdx.x][0];
}

// ------------------------------------------------------ init / read

template <class L, typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_init(FieldArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    R h[L::Q];
    R g[L::QT];
    if (a.mask && (a.mask[cell] & MASK_SOLID)) {
        const R nan = (R)__builtin_nan("");
#pragma unroll
        for (int q = 0; q < L::Q; ++q) h[q] = nan;
#pragma unroll
        for (int k = 0; k < L::QT; ++k) g[k] = nan;
    } else {
        const int64_t n = G.ncell;  // the velocity planes u[k * n + cell] reach 3 n > 2^31
        const R T = (TH && a.T) ? a.T[cell] : R(0);
        equilibrium<R, TH>(a.rho[cell], a.u[cell], a.u[n + cell], a.u[2 * n + cell], T, a.col.a_T, h, g);
    }
#pragma unroll
    for (int q = 0; q < L::Q; ++q) st(a.f, posf(G, q, cell), h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < L::QT; ++k) st(a.g, posg(G, k, cell), g[k]);
    }
}

// Populations of `cell` at the current time: after an even number of steps
// (or with two buffers) in the cell's own slots, after an odd number where
// the last odd step stored them, (opposite(q), x - c_q), with in-kernel
// bounce-back's re-read of blocked inflows.  Returns false for a solid cell.
template <class L, typename R, bool TH>
__device__ __forceinline__ bool load_cell(const FieldArgs<R>& a, int32_t cell, R* h, R* g)
{
    const Geometry& G = a.geo;
    if (a.ab || a.parity == 0) {
#pragma unroll
        for (int q = 0; q < L::Q; ++q) h[q] = ld(a.f, posf(G, q, cell));
        if (TH) {
#pragma unroll
            for (int k = 0; k < L::QT; ++k) g[k] = ld(a.g, posg(G, k, cell));
        }
    } else {
        const Nbr<L::DIMS> nb(G, cell);
#pragma unroll
        for (int q = 0; q < L::Q; ++q) h[q] = ld(a.f, posf(G, opp(q), cell + nb.at(-L::cx(q), -L::cy(q), -L::cz(q))));
        if (TH) {
#pragma unroll
            for (int k = 0; k < L::QT; ++k)
                g[k] = ld(a.g, posg(G, opp(k), cell + nb.at(-L::cxT(k), -L::cyT(k), -L::czT(k))));
        }
        // with in-kernel boundary rules, an inflow from across a face or a
        // solid is the returning population the even step left behind
        if (a.bb.in_kernel) {
            const Blocked b = blocked_dirs<L>(a.bb, a.mask, cell, nb.faces);
            const uint32_t blk = b.is_solid ? 0u : (b.wall | b.solid);
            if (blk != 0) {
                const FaceRules fr = face_rules<L>(a.bb, nb.faces);
#pragma unroll
                for (int q = 1; q < L::Q; ++q)
                    if ((blk >> opp(q)) & 1u) h[q] = blocked_inflow<L, R, 2>(a.f, G, cell, nb, fr, a.bb, q);
                if (TH) {
#pragma unroll
                    for (int k = 1; k < L::QT; ++k)
                        if ((blk >> opp(k)) & 1u) g[k] = bounce7(a.bb, b, opp(k), ld(a.g, posg(G, k, cell)));
                }
            }
        }
    }
    return !(a.mask && (a.mask[cell] & MASK_SOLID));
}

template <typename R>
__device__ __forceinline__ bool finite_macros(const Macro<R>& m)
{
    return __builtin_isfinite(m.rho) && __builtin_isfinite(m.T) && __builtin_isfinite(m.ux) &&
           __builtin_isfinite(m.uy) && __builtin_isfinite(m.uz);
}

template <class L, typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_read(FieldArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t n = G.ncell;  // the velocity planes u_out[k * n + cell] reach 3 n > 2^31
    R h[L::Q];
    R g[L::QT];
    Macro<R> m;
    if (!load_cell<L, R, TH>(a, cell, h, g)) {
        const R nan = (R)__builtin_nan("");
        m.rho = m.ux = m.uy = m.uz = m.T = nan;
    } else {
        m = macros<R, TH>(h, g, a.col);
        if (!finite_macros(m)) atomicOr(a.unstable, 1);
    }
    if (a.rho_out) a.rho_out[cell] = m.rho;
    if (a.u_out) {
        a.u_out[cell] = m.ux;
        a.u_out[n + cell] = m.uy;
        a.u_out[2 * n + cell] = m.uz;
    }
    if (TH && a.T_out) a.T_out[cell] = m.T;
}

// Sums over the fluid cells at the current time, in fp64: the cell count,
// mass, momentum rho u, kinetic energy rho |u|^2 / 2, the largest |u|^2,
// heat T and the advective heat flux u T (u with the half force, as in the
// read-back).  Grid-stride over cells; wavefront shuffles, then LDS across
// the block's wavefronts, then one global atomic per block and value (the
// maximum through the ordering of non-negative doubles' bit patterns).
template <class L, typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_diag(FieldArgs<R> a, double* out)
{
    constexpr int NS = LBM_DIAG_COUNT;  // slot LBM_DIAG_UMAX holds max |u|^2
    __shared__ double part[BLOCK / 64][NS];
    double acc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[i] = 0.0;
    const int32_t n = a.geo.ncell;
    for (int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x); cell < n;
         cell += (int32_t)(gridDim.x * BLOCK)) {
        R h[L::Q];
        R g[L::QT];
        if (!load_cell<L, R, TH>(a, cell, h, g)) continue;
        const Macro<R> m = macros<R, TH>(h, g, a.col);
        if (!finite_macros(m)) atomicOr(a.unstable, 1);
        const double rho = m.rho, ux = m.ux, uy = m.uy, uz = m.uz, T = TH ? (double)m.T : 0.0;
        const double u2 = ux * ux + uy * uy + uz * uz;
        acc[LBM_DIAG_FLUID_CELLS] += 1.0;
        acc[LBM_DIAG_MASS] += rho;
        acc[LBM_DIAG_MOM_X] += rho * ux;
        acc[LBM_DIAG_MOM_Y] += rho * uy;
        acc[LBM_DIAG_MOM_Z] += rho * uz;
        acc[LBM_DIAG_KINETIC] += 0.5 * rho * u2;
        acc[LBM_DIAG_UMAX] = (u2 > acc[LBM_DIAG_UMAX] || u2 != u2) ? u2 : acc[LBM_DIAG_UMAX];
        acc[LBM_DIAG_HEAT] += T;
        acc[LBM_DIAG_CONV_X] += ux * T;
        acc[LBM_DIAG_CONV_Y] += uy * T;
        acc[LBM_DIAG_CONV_Z] += uz * T;
    }
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        double v = acc[i];
        if (i == LBM_DIAG_UMAX) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const double w = __shfl_xor(v, o, 64);
                v = (w > v || w != w) ? w : v;
            }
        } else {
            v = wave_sum(v);
        }
        if ((threadIdx.x & 63) == 0) part[wave][i] = v;
    }
    __syncthreads();
    if (threadIdx.x < NS) {
        const int i = threadIdx.x;
        double v = part[0][i];
        for (int w = 1; w < BLOCK / 64; ++w) {
            const double x = part[w][i];
            if (i == LBM_DIAG_UMAX) v = (x > v || x != x) ? x : v;
            else v += x;
        }
        if (i == LBM_DIAG_UMAX) {
            // a non-negative double (or NaN) orders like its bit pattern
            atomicMax(reinterpret_cast<unsigned long long*>(out + i), (unsigned long long)__double_as_longlong(v));
        } else if (v != 0.0) {
            atomicAdd(out + i, v);
        }
    }
}

__global__ void __launch_bounds__(BLOCK) k_zero_f64(double* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (i < n) p[i] = 0.0;
}

// Every 32-bit word of [p, p + 16 n16 bytes) set to `word`.  Grid-stride
// over 16-byte words.
__global__ void __launch_bounds__(BLOCK) k_fill_words(uint4* p, int64_t n16, uint32_t word)
{
    const uint4 v = make_uint4(word, word, word, word);
    for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < n16; i += (int64_t)gridDim.x * BLOCK) p[i] = v;
}

inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + BLOCK - 1) / BLOCK)); }

}  // namespace

// One launch of a cell kernel over the whole box.  A reservation of more
// than 64 KiB of local data share needs the kernel's limit raised first.
template <auto K, typename A>
hipError_t launch_cells(const A& a, size_t lds, hipStream_t s)
{
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)K, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(K, grid_for(a.geo.ncell), dim3(BLOCK), lds, s, a);
    return hipGetLastError();
}

// Pick the <thermal, boundary rules> instance of a cell kernel: no in-kernel
// boundary, walls and solids only, or also SLIP / VELOCITY / PRESSURE faces.
#define LBM_CELL_LAUNCH(KERNEL, a, thermal, lds, s)                                       \
    do {                                                                                  \
        const int bnd_ = boundary_rules((a).bb);                                          \
        if (thermal) {                                                                    \
            if (bnd_ == 2) return launch_cells<KERNEL<L, R, true, 2>>(a, lds, s);         \
            if (bnd_ == 1) return launch_cells<KERNEL<L, R, true, 1>>(a, lds, s);         \
            return launch_cells<KERNEL<L, R, true, 0>>(a, lds, s);                        \
        }                                                                                 \
        if (bnd_ == 2) return launch_cells<KERNEL<L, R, false, 2>>(a, lds, s);            \
        if (bnd_ == 1) return launch_cells<KERNEL<L, R, false, 1>>(a, lds, s);            \
        return launch_cells<KERNEL<L, R, false, 0>>(a, lds, s);                           \
    } while (0)

template <class L, typename R>
hipError_t launch_aa_step(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_aa_step, a, thermal, lds, s);
}

template <class L, typename R>
hipError_t launch_ab_collide(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_ab_collide, a, thermal, lds, s);
}

template <class L, typename R>
hipError_t launch_ab_pull(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_ab_pull, a, thermal, lds, s);
}

template <class L, typename R>
hipError_t launch_ab_push(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_ab_push, a, thermal, lds, s);
}

template <typename R>
hipError_t launch_link_gather(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.end <= a.begin) return hipSuccess;
    hipLaunchKernelGGL((k_link_gather<R>), grid_for(a.end - a.begin), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_link_scatter(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.end <= a.begin) return hipSuccess;
    hipLaunchKernelGGL((k_link_scatter<R>), grid_for(a.end - a.begin), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_link_direct(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.end <= a.begin) return hipSuccess;
    hipLaunchKernelGGL((k_link_direct<R>), grid_for(a.end - a.begin), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <class L, typename R>
hipError_t launch_link_force(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.n_seg > 0) {
        const int64_t waves = BLOCK / 64;
        hipLaunchKernelGGL((k_link_force<L, R>), dim3((unsigned)((a.n_seg + waves - 1) / waves)), dim3(BLOCK), 0, s,
                           a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_force_groups, dim3(LBM_GROUPS), dim3(BLOCK), 0, s, a.group_seg, (const double*)a.seg_sum,
                       a.accum);
    return hipGetLastError();
}

template <class L, typename R>
hipError_t launch_init(const FieldArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_init<L, R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_init<L, R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <class L, typename R>
hipError_t launch_read(const FieldArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_read<L, R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_read<L, R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <class L, typename R>
hipError_t launch_diag(const FieldArgs<R>& a, bool thermal, double* out, hipStream_t s)
{
    const unsigned blocks = (unsigned)std::min<int64_t>(((int64_t)a.geo.ncell + BLOCK - 1) / BLOCK, 2048);
    if (thermal) hipLaunchKernelGGL((k_diag<L, R, true>), dim3(blocks), dim3(BLOCK), 0, s, a, out);
    else hipLaunchKernelGGL((k_diag<L, R, false>), dim3(blocks), dim3(BLOCK), 0, s, a, out);
    return hipGetLastError();
}

hipError_t launch_zero_f64(double* p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_f64, grid_for(n), dim3(BLOCK), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_words(void* p, size_t bytes, uint32_t word, hipStream_t s)
{
    if (((uintptr_t)p | bytes) & 15u) return hipErrorInvalidValue;
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n16 + BLOCK - 1) / BLOCK, 65536);
    hipLaunchKernelGGL(k_fill_words, dim3((unsigned)blocks), dim3(BLOCK), 0, s, (uint4*)p, n16, word);
    return hipGetLastError();
}

#define LBM_INSTANTIATE_LATTICE(L, R)                                                      \
    template hipError_t launch_aa_step<L, R>(const StepArgs<R>&, bool, size_t, hipStream_t);    \
    template hipError_t launch_ab_collide<L, R>(const StepArgs<R>&, bool, size_t, hipStream_t); \
    template hipError_t launch_ab_pull<L, R>(const StepArgs<R>&, bool, size_t, hipStream_t);    \
    template hipError_t launch_ab_push<L, R>(const StepArgs<R>&, bool, size_t, hipStream_t);    \
    template hipError_t launch_link_force<L, R>(const LinkArgs<R>&, hipStream_t);          \
    template hipError_t launch_init<L, R>(const FieldArgs<R>&, bool, hipStream_t);         \
    template hipError_t launch_read<L, R>(const FieldArgs<R>&, bool, hipStream_t);         \
    template hipError_t launch_diag<L, R>(const FieldArgs<R>&, bool, double*, hipStream_t);
#define LBM_INSTANTIATE(R)                                                                 \
    template hipError_t launch_link_gather<R>(const LinkArgs<R>&, hipStream_t);            \
    template hipError_t launch_link_scatter<R>(const LinkArgs<R>&, hipStream_t);           \
    template hipError_t launch_link_direct<R>(const LinkArgs<R>&, hipStream_t);            \
    LBM_INSTANTIATE_LATTICE(Lat3D, R)                                                      \
    LBM_INSTANTIATE_LATTICE(Lat2D, R)

LBM_INSTANTIATE(float)
LBM_INSTANTIATE(double)

}  // namespace lbm
