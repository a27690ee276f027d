// lbm_kernels.hip -- the HIP kernels of the fused lattice Boltzmann step (gfx950).
//
// Layout: structure of arrays, one plane of `stride` elements per population
// direction, cell index x + nx*(y + ny*z) inside a plane ("Multi-GPU thermal
// lattice Boltzmann simulations using OpenACC and MPI", Sec. 3: SoA so that
// neighbouring threads touch neighbouring data).  One thread per cell, cells
// flattened, so a 64-lane wavefront reads and writes 64 consecutive elements
// of each plane (256 B in fp32) whatever the box shape.
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

// Run-time direction tables packed into 64-bit constants: 2 bits per
// direction holding c + 1.
__host__ __device__ constexpr uint64_t pack_dirs(int which, int Q)
{
    uint64_t v = 0;
    for (int q = 0; q < Q; ++q) {
        int c = 0;
        if (Q == Q19) c = which == 0 ? cx19(q) : (which == 1 ? cy19(q) : cz19(q));
        else c = which == 0 ? cx7(q) : (which == 1 ? cy7(q) : cz7(q));
        v |= (uint64_t)(c + 1) << (2 * q);
    }
    return v;
}
constexpr uint64_t CX19 = pack_dirs(0, Q19), CY19 = pack_dirs(1, Q19), CZ19 = pack_dirs(2, Q19);

__device__ __forceinline__ int dir_comp(uint64_t packed, int q) { return (int)((packed >> (2 * q)) & 3u) - 1; }
__device__ __forceinline__ int opp_rt(int q) { return q == 0 ? 0 : ((q & 1) ? q + 1 : q - 1); }
__device__ __forceinline__ double w19_rt(int q) { return q == 0 ? 1.0 / 3.0 : (q <= 6 ? 1.0 / 18.0 : 1.0 / 36.0); }

// Wrapped neighbour offsets of one cell: a cell's coordinates are computed
// once and each axis wraps with a compare and an add.
struct Nbr {
    int32_t xm, xp, ym, yp, zm, zp;
    uint32_t faces;  // bit f: the cell touches box face f (x-, x+, y-, y+, z-, z+)

    __device__ __forceinline__ Nbr(const Geometry& G, int32_t cell)
    {
        const uint32_t r = divide((uint32_t)cell, G.div_nx);
        const int32_t x = cell - (int32_t)r * G.nx;
        const uint32_t z = divide(r, G.div_ny);
        const int32_t y = (int32_t)r - (int32_t)z * G.ny;
        xm = (x == 0) ? G.nx - 1 : -1;
        xp = (x == G.nx - 1) ? 1 - G.nx : 1;
        ym = (y == 0) ? (G.ny - 1) * G.nx : -G.nx;
        yp = (y == G.ny - 1) ? (1 - G.ny) * G.nx : G.nx;
        zm = ((int32_t)z == 0) ? (G.nz - 1) * G.nxy : -G.nxy;
        zp = ((int32_t)z == G.nz - 1) ? (1 - G.nz) * G.nxy : G.nxy;
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

// Element `idx` of a population plane.  The plane base is uniform across the
// wavefront (a scalar register) and the byte offset is a 32-bit unsigned
// value, so loads and stores take the scalar-base + 32-bit-offset addressing
// form instead of a 64-bit address per lane.  Requires stride * sizeof(R) <
// 2^32 (checked on the host).
template <typename R>
__device__ __forceinline__ R ld(const R* plane, int32_t idx)
{
    return *reinterpret_cast<const R*>(reinterpret_cast<const char*>(plane) + (uint32_t)idx * (uint32_t)sizeof(R));
}
template <typename R>
__device__ __forceinline__ void st(R* plane, int32_t idx, R v)
{
    *reinterpret_cast<R*>(reinterpret_cast<char*>(plane) + (uint32_t)idx * (uint32_t)sizeof(R)) = v;
}

// ------------------------------------------------------ boundaries

// D3Q19 directions leaving the box through face f (x-, x+, y-, y+, z-, z+).
__host__ __device__ constexpr uint32_t dirs_through(int f)
{
    uint32_t m = 0;
    for (int q = 1; q < Q19; ++q) {
        const int c = (f >> 1) == 0 ? cx19(q) : ((f >> 1) == 1 ? cy19(q) : cz19(q));
        if ((f & 1) ? c > 0 : c < 0) m |= 1u << q;
    }
    return m;
}

// Face crossed by D3Q7 direction k (1..6).
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

template <typename R>
__device__ __forceinline__ Blocked blocked_dirs(const Bounce<R>& bb, const uint32_t* mask, int32_t cell,
                                                uint32_t faces)
{
    Blocked b;
    const uint32_t fw = faces & (uint32_t)bb.walls;
    b.wall = ((fw & 1u) ? dirs_through(0) : 0u) | ((fw & 2u) ? dirs_through(1) : 0u) |
             ((fw & 4u) ? dirs_through(2) : 0u) | ((fw & 8u) ? dirs_through(3) : 0u) |
             ((fw & 16u) ? dirs_through(4) : 0u) | ((fw & 32u) ? dirs_through(5) : 0u);
    const uint32_t m = mask ? mask[cell] : 0u;
    b.is_solid = (m & MASK_SOLID) != 0;
    b.solid = b.is_solid ? 0u : m;
    b.claim = b.is_solid ? (m & ~MASK_SOLID) : 0u;
    return b;
}

// The value a D3Q7 population takes when it bounces in direction k's face or
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

// ------------------------------------------------------------ AA step


// One fused time step in place.  With BND the step also applies half-way
// bounce-back at no-slip walls and solid cells ("Multi-GPU thermal lattice
// Boltzmann simulations using OpenACC and MPI", Sec. 2); without it the box
// streams as if periodic and link passes fix the blocked directions.
// All bounce-back work happens in the odd step; the even step is the plain
// kernel for every cell (solid cells compute on NaN in their own slots):
//  * even step: every cell stores f_p^+ at (opp p, x);
//  * odd step, inflow: a population q whose upstream cell x - c_q is across
//    a wall or solid is the bounce of f_opp(q)^+(x) from the even step, which
//    sits in (q, x) of the cell itself -- it is read there;
//  * odd step, outflow: f_p^+ for a blocked direction p is stored at
//    (opp p, x), where the next (even) step reads it.  Its usual slot is
//    skipped when p leaves through a wall (the addressing wraps onto the cell
//    across the box, whose slot that is) and kept when p points at a solid
//    cell (only that solid cell reads it next).
// A solid cell skips its odd-step stores into slots a fluid neighbour claims
// this way (mask bits) and into wrapped slots across a wall.  No slot is
// touched by two cells in one step.
template <typename R, bool TH, bool BND>
__global__ void __launch_bounds__(BLOCK) k_aa_step(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    R* __restrict__ f = a.f;
    R* __restrict__ gg = a.g;
    R h[Q19];
    R g[Q7];
    if (a.parity == 0) {
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = ld(f + q * S, cell);
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) g[k] = ld(gg + k * S, cell);
        }
        collide<R, TH>(h, g, a.col);
#pragma unroll
        for (int q = 0; q < Q19; ++q) st(f + opp19(q) * S, cell, h[q]);
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) st(gg + opp7(k) * S, cell, g[k]);
        }
        return;
    }
    const Nbr nb(G, cell);
    Blocked b{0u, 0u, 0u, false};
    if (BND) b = blocked_dirs(a.bb, a.mask, cell, nb.faces);
    const uint32_t blk = b.wall | b.solid;           // a fluid cell's bounced directions
    const uint32_t skip = b.wall | b.claim;          // usual odd-step stores to leave out
    const bool near = BND && !b.is_solid && blk != 0;
#pragma unroll
    for (int q = 0; q < Q19; ++q) h[q] = ld(f + opp19(q) * S, cell + nb.at(-cx19(q), -cy19(q), -cz19(q)));
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) g[k] = ld(gg + opp7(k) * S, cell + nb.at(-cx7(k), -cy7(k), -cz7(k)));
    }
    if (near) {
#pragma unroll
        for (int q = 1; q < Q19; ++q)
            if ((blk >> opp19(q)) & 1u) h[q] = ld(f + q * S, cell);
        if (TH) {
#pragma unroll
            for (int k = 1; k < Q7; ++k)
                if ((blk >> opp7(k)) & 1u) g[k] = bounce7(a.bb, b, opp7(k), ld(gg + k * S, cell));
        }
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < Q19; ++q)
        if (!BND || !((skip >> q) & 1u)) st(f + q * S, cell + nb.at(cx19(q), cy19(q), cz19(q)), h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k)
            if (!BND || !((skip >> k) & 1u)) st(gg + k * S, cell + nb.at(cx7(k), cy7(k), cz7(k)), g[k]);
    }
    if (near) {
#pragma unroll
        for (int q = 1; q < Q19; ++q)
            if ((blk >> q) & 1u) st(f + opp19(q) * S, cell, h[q]);
        if (TH) {
#pragma unroll
            for (int k = 1; k < Q7; ++k)
                if ((blk >> k) & 1u) st(gg + opp7(k) * S, cell, bounce7(a.bb, b, k, g[k]));
        }
    }
}

// ------------------------------------------------- two buffers (A-B)

// Collide in place: every population stays in its own slot (solid cells
// compute on NaN in theirs; no fluid cell pulls from a solid slot).
template <typename R, bool TH, bool BND>
__global__ void __launch_bounds__(BLOCK) k_ab_collide(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    R h[Q19];
    R g[Q7];
#pragma unroll
    for (int q = 0; q < Q19; ++q) h[q] = ld(a.f + q * S, cell);
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) g[k] = ld(a.g + k * S, cell);
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < Q19; ++q) st(a.f + q * S, cell, h[q]);
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) st(a.g + k * S, cell, g[k]);
    }
}

// Pull into the other buffer: B(q, x) = A(q, x - c_q).  With BND, when
// x - c_q is across a wall or a solid cell the population comes back from x
// itself: B(q, x) = A(opp q, x) (anti-bounce-back for a Dirichlet D3Q7 one).
template <typename R, bool TH, bool BND>
__global__ void __launch_bounds__(BLOCK) k_ab_pull(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    const Nbr nb(G, cell);
    Blocked b{0u, 0u, 0u, false};
    if (BND) b = blocked_dirs(a.bb, a.mask, cell, nb.faces);
    const uint32_t blk = b.is_solid ? 0u : (b.wall | b.solid);
#pragma unroll
    for (int q = 0; q < Q19; ++q) {
        R v = ld(a.f + q * S, cell + nb.at(-cx19(q), -cy19(q), -cz19(q)));
        if (BND && ((blk >> opp19(q)) & 1u)) v = ld(a.f + opp19(q) * S, cell);
        st(a.f2 + q * S, cell, v);
    }
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) {
            R v = ld(a.g + k * S, cell + nb.at(-cx7(k), -cy7(k), -cz7(k)));
            if (BND && ((blk >> opp7(k)) & 1u)) v = bounce7(a.bb, b, opp7(k), ld(a.g + opp7(k) * S, cell));
            st(a.g2 + k * S, cell, v);
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
        s.src_plane = opp_rt(p);
        s.src_idx = cell;
        s.dst_plane = p;
        s.dst_idx = cellw;
    } else if (mode == LINK_AA_AFTER_ODD) {
        s.src_plane = p;
        s.src_idx = cellw;
        s.dst_plane = opp_rt(p);
        s.dst_idx = cell;
    } else {
        s.src_plane = p;
        s.src_idx = cell;
        s.dst_plane = opp_rt(p);
        s.dst_idx = cell;
    }
    return s;
}

// Per-link contribution to the group sums: the wall receives 2 c_p f_p^+
// (D3Q19; the stored value is f - w), and a Dirichlet D3Q7 link passes
// w T_w - 2 g_p^+ into the fluid.
struct LinkSum {
    double fx, fy, fz, q;
};

template <typename R>
__device__ __forceinline__ LinkSum link_sum(const LinkArgs<R>& a, uint32_t meta, int p, int32_t grp, R v)
{
    LinkSum c{0.0, 0.0, 0.0, 0.0};
    if (!(meta & LINK_D3Q7)) {
        const double fv = 2.0 * ((double)v + w19_rt(p));
        c.fx = dir_comp(CX19, p) * fv;
        c.fy = dir_comp(CY19, p) * fv;
        c.fz = dir_comp(CZ19, p) * fv;
    } else if (meta & LINK_DIRICHLET) {
        c.q = a.omega * a.wall_T[grp] - 2.0 * (double)v;
    }
    return c;
}

// Value a link writes: bounce-back f_pbar = f_p^+ (no-slip), anti-bounce-back
// g_pbar = -g_p^+ + w T_w (Dirichlet T), bounce-back g_pbar = g_p^+ (adiabatic).
template <typename R>
__device__ __forceinline__ R link_value(const LinkArgs<R>& a, uint32_t meta, int32_t grp, R v)
{
    if ((meta & LINK_D3Q7) && (meta & LINK_DIRICHLET)) return (R)(a.omega * a.wall_T[grp]) - v;
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
    const int64_t S = a.geo.stride;
    const uint32_t meta = a.meta[l];
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    const R* src = (meta & LINK_D3Q7) ? a.g_src : a.f_src;
    a.scratch[l] = ld(src + sl.src_plane * S, sl.src_idx);
}

// Scatter (wall links): write each gathered value where the next step reads it.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_scatter(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const int64_t S = a.geo.stride;
    const uint32_t meta = a.meta[l];
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    R* dst = (meta & LINK_D3Q7) ? a.g_dst : a.f_dst;
    st(dst + sl.dst_plane * S, sl.dst_idx, link_value(a, meta, grp, a.scratch[l]));
}

// Direct pass (wall links with two buffers): sources lie in one buffer and
// destinations in the other, so gather and scatter merge into one pass.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_direct(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const int64_t S = a.geo.stride;
    const uint32_t meta = a.meta[l];
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const LinkSlots sl = link_slots(a.mode, (int)(meta & LINK_DIR_MASK), a.cell[l], a.cellw[l]);
    const bool g7 = (meta & LINK_D3Q7) != 0;
    const R v = ld((g7 ? a.g_src : a.f_src) + sl.src_plane * S, sl.src_idx);
    st((g7 ? a.g_dst : a.f_dst) + sl.dst_plane * S, sl.dst_idx, link_value(a, meta, grp, v));
}

// Force pass, on a submission's last step only, over every link.  It reads
// the bounced population f_p^+ of each link where the step left it: with
// in-kernel bounce-back (opp p, x) in place (the even step's usual store or
// the odd step's bounce-back store); with link passes the scatter
// destination; with two buffers B(opp p, x).  Values a D3Q7 Dirichlet link stores after
// anti-bounce-back are converted back.  It sums the momentum exchange
// 2 c_p f_p^+ and the heat w T_w - 2 g_p^+ per group: wavefront shuffles, then
// fp64 LDS atomics per block, then one global atomic per block and touched
// group; a grid-stride loop keeps the block count (and the global atomics)
// small.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_force(LinkArgs<R> a)
{
    __shared__ double acc[4 * LBM_GROUPS];
    for (int i = threadIdx.x; i < 4 * LBM_GROUPS; i += BLOCK) acc[i] = 0.0;
    __syncthreads();
    const int64_t S = a.geo.stride;
    for (int64_t base = a.begin + (int64_t)blockIdx.x * BLOCK; base < a.end; base += (int64_t)gridDim.x * BLOCK) {
        const int64_t l = base + threadIdx.x;
        LinkSum c{0.0, 0.0, 0.0, 0.0};
        int32_t grp = -1;
        if (l < a.end) {
            const uint32_t meta = a.meta[l];
            const int p = (int)(meta & LINK_DIR_MASK);
            grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
            const bool g7 = (meta & LINK_D3Q7) != 0;
            int32_t plane, idx;
            bool transformed;
            if (a.in_kernel && a.mode != LINK_AB) {
                // even step: the usual store; odd step: the bounce-back store
                plane = opp_rt(p);
                idx = a.cell[l];
                transformed = a.mode == LINK_AA_AFTER_ODD;
            } else {
                // link passes, or the two-buffer pull: the link's destination
                const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
                plane = sl.dst_plane;
                idx = sl.dst_idx;
                transformed = true;
            }
            R v = ld((g7 ? a.g_dst : a.f_dst) + plane * S, idx);
            if (transformed && g7 && (meta & LINK_DIRICHLET)) v = (R)(a.omega * a.wall_T[grp]) - v;
            c = link_sum(a, meta, p, grp, v);
        }
        const int32_t lead = __shfl(grp, 0, 64);
        if (__all(grp == lead || grp < 0)) {
            c.fx = wave_sum(c.fx);
            c.fy = wave_sum(c.fy);
            c.fz = wave_sum(c.fz);
            c.q = wave_sum(c.q);
            if ((threadIdx.x & 63) == 0 && lead >= 0) {
                atomicAdd(&acc[4 * lead + 0], c.fx);
                atomicAdd(&acc[4 * lead + 1], c.fy);
                atomicAdd(&acc[4 * lead + 2], c.fz);
                atomicAdd(&acc[4 * lead + 3], c.q);
            }
        } else if (grp >= 0) {
            atomicAdd(&acc[4 * grp + 0], c.fx);
            atomicAdd(&acc[4 * grp + 1], c.fy);
            atomicAdd(&acc[4 * grp + 2], c.fz);
            atomicAdd(&acc[4 * grp + 3], c.q);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * LBM_GROUPS; i += BLOCK)
        if (acc[i] != 0.0) atomicAdd(a.accum + i, acc[i]);
}

// ------------------------------------------------------ init / read

template <typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_init(FieldArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    R h[Q19];
    R g[Q7];
    if (a.mask && (a.mask[cell] & MASK_SOLID)) {
        const R nan = (R)__builtin_nan("");
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = nan;
#pragma unroll
        for (int k = 0; k < Q7; ++k) g[k] = nan;
    } else {
        const int32_t n = G.ncell;
        const R T = (TH && a.T) ? a.T[cell] : R(0);
        equilibrium<R, TH>(a.rho[cell], a.u[cell], a.u[n + cell], a.u[2 * n + cell], T, a.col.a_T, h, g);
    }
#pragma unroll
    for (int q = 0; q < Q19; ++q) a.f[q * S + cell] = h[q];
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) a.g[k * S + cell] = g[k];
    }
}

// Populations of `cell` at the current time: after an even number of steps
// (or with two buffers) in the cell's own slots, after an odd number where
// the last odd step stored them, (opposite(q), x - c_q), with in-kernel
// bounce-back's re-read of blocked inflows.  Returns false for a solid cell.
template <typename R, bool TH>
__device__ __forceinline__ bool load_cell(const FieldArgs<R>& a, int32_t cell, R* h, R* g)
{
    const Geometry& G = a.geo;
    const int64_t S = G.stride;
    if (a.ab || a.parity == 0) {
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = a.f[q * S + cell];
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) g[k] = a.g[k * S + cell];
        }
    } else {
        const Nbr nb(G, cell);
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = a.f[opp19(q) * S + (cell + nb.at(-cx19(q), -cy19(q), -cz19(q)))];
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) g[k] = a.g[opp7(k) * S + (cell + nb.at(-cx7(k), -cy7(k), -cz7(k)))];
        }
        // with in-kernel bounce-back, an inflow from across a wall or a solid
        // is the bounce of the cell's own even-step output, kept in (q, x)
        if (a.bb.in_kernel) {
            const Blocked b = blocked_dirs(a.bb, a.mask, cell, nb.faces);
            const uint32_t blk = b.is_solid ? 0u : (b.wall | b.solid);
            if (blk != 0) {
#pragma unroll
                for (int q = 1; q < Q19; ++q)
                    if ((blk >> opp19(q)) & 1u) h[q] = a.f[q * S + cell];
                if (TH) {
#pragma unroll
                    for (int k = 1; k < Q7; ++k)
                        if ((blk >> opp7(k)) & 1u) g[k] = bounce7(a.bb, b, opp7(k), a.g[k * S + cell]);
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

template <typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_read(FieldArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int32_t n = G.ncell;
    R h[Q19];
    R g[Q7];
    Macro<R> m;
    if (!load_cell<R, TH>(a, cell, h, g)) {
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
template <typename R, bool TH>
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
        R h[Q19];
        R g[Q7];
        if (!load_cell<R, TH>(a, cell, h, g)) continue;
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

inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + BLOCK - 1) / BLOCK)); }

}  // namespace

// Pick the <thermal, in-kernel bounce-back> instance of a cell kernel.
#define LBM_CELL_LAUNCH(KERNEL, a, thermal, s)                                                              \
    do {                                                                                                    \
        const dim3 grid_ = grid_for((a).geo.ncell);                                                         \
        const bool solid_ = (a).bb.in_kernel != 0;                                                          \
        if (thermal && solid_) hipLaunchKernelGGL((KERNEL<R, true, true>), grid_, dim3(BLOCK), 0, s, a);    \
        else if (thermal) hipLaunchKernelGGL((KERNEL<R, true, false>), grid_, dim3(BLOCK), 0, s, a);        \
        else if (solid_) hipLaunchKernelGGL((KERNEL<R, false, true>), grid_, dim3(BLOCK), 0, s, a);         \
        else hipLaunchKernelGGL((KERNEL<R, false, false>), grid_, dim3(BLOCK), 0, s, a);                    \
    } while (0)

template <typename R>
hipError_t launch_aa_step(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_aa_step, a, thermal, s);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_ab_collide(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_ab_collide, a, thermal, s);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_ab_pull(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    LBM_CELL_LAUNCH(k_ab_pull, a, thermal, s);
    return hipGetLastError();
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

template <typename R>
hipError_t launch_link_force(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.end <= a.begin) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((a.end - a.begin + BLOCK - 1) / BLOCK, 1024);
    hipLaunchKernelGGL((k_link_force<R>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_init(const FieldArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_init<R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_init<R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_read(const FieldArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_read<R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_read<R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_diag(const FieldArgs<R>& a, bool thermal, double* out, hipStream_t s)
{
    const unsigned blocks = (unsigned)std::min<int64_t>(((int64_t)a.geo.ncell + BLOCK - 1) / BLOCK, 2048);
    if (thermal) hipLaunchKernelGGL((k_diag<R, true>), dim3(blocks), dim3(BLOCK), 0, s, a, out);
    else hipLaunchKernelGGL((k_diag<R, false>), dim3(blocks), dim3(BLOCK), 0, s, a, out);
    return hipGetLastError();
}

hipError_t launch_zero_f64(double* p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_f64, grid_for(n), dim3(BLOCK), 0, s, p, n);
    return hipGetLastError();
}

#define LBM_INSTANTIATE(R)                                                               \
    template hipError_t launch_aa_step<R>(const StepArgs<R>&, bool, hipStream_t);        \
    template hipError_t launch_ab_collide<R>(const StepArgs<R>&, bool, hipStream_t);     \
    template hipError_t launch_ab_pull<R>(const StepArgs<R>&, bool, hipStream_t);        \
    template hipError_t launch_link_gather<R>(const LinkArgs<R>&, hipStream_t);          \
    template hipError_t launch_link_scatter<R>(const LinkArgs<R>&, hipStream_t);         \
    template hipError_t launch_link_direct<R>(const LinkArgs<R>&, hipStream_t);          \
    template hipError_t launch_link_force<R>(const LinkArgs<R>&, hipStream_t);           \
    template hipError_t launch_init<R>(const FieldArgs<R>&, bool, hipStream_t);          \
    template hipError_t launch_read<R>(const FieldArgs<R>&, bool, hipStream_t);          \
    template hipError_t launch_diag<R>(const FieldArgs<R>&, bool, double*, hipStream_t);

LBM_INSTANTIATE(float)
LBM_INSTANTIATE(double)

}  // namespace lbm
