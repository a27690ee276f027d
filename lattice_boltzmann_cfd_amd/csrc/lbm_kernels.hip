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
// are processed like fluid ones (they hold NaN); every slot they write is
// overwritten by a link scatter before any fluid cell reads it.
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

// ------------------------------------------------------------ AA step

// Value a D3Q7 population takes when it bounces off a solid cell:
// anti-bounce-back -g^+ + w T_solid (Dirichlet) or g^+ (adiabatic).
template <typename R>
__device__ __forceinline__ R solid_rule(const StepArgs<R>& a, R v)
{
    return a.solid_dirichlet ? a.solid_gw - v : v;
}

// One fused time step in place.  With SOLID the fluid cells next to solid
// cells apply half-way bounce-back themselves ("Multi-GPU thermal lattice
// Boltzmann simulations using OpenACC and MPI", Sec. 2), and all of it happens
// in the odd step, so the even step stays the plain kernel for every cell:
//  * even step: each cell stores f_p^+ at (opp p, x) as usual, solid cells
//    included (on NaN; nobody reads a solid cell's slots in the odd step);
//  * odd step, inflow: a population q whose upstream cell x - c_q is solid is
//    the bounce of f_opp(q)^+(x) from the even step, which sits in (q, x) of
//    the cell itself -- it is read there instead;
//  * odd step, outflow: f_p^+ for a direction p that points at a solid cell is
//    stored, besides its usual slot (read next only by the solid cell), at
//    (opp p, x), where the next (even) step reads it.
// A solid cell's usual odd-step store of direction q lands in (q, s + c_q);
// when s + c_q is a fluid cell bouncing off s that slot is the fluid cell's
// re-read and bounce-back slot, so the solid cell skips it (its mask bit q).
// No other slot is touched by two cells in one step.
template <typename R, bool TH, bool SOLID>
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
    } else {
        const uint32_t m = SOLID ? a.mask[cell] : 0u;
        const bool solid = SOLID && (m & MASK_SOLID);
        const bool near = SOLID && !solid && m != 0;
        const Nbr nb(G, cell);
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = ld(f + opp19(q) * S, cell + nb.at(-cx19(q), -cy19(q), -cz19(q)));
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) g[k] = ld(gg + opp7(k) * S, cell + nb.at(-cx7(k), -cy7(k), -cz7(k)));
        }
        if (near) {
#pragma unroll
            for (int q = 1; q < Q19; ++q)
                if ((m >> opp19(q)) & 1u) h[q] = ld(f + q * S, cell);
            if (TH) {
#pragma unroll
                for (int k = 1; k < Q7; ++k)
                    if ((m >> opp7(k)) & 1u) g[k] = solid_rule(a, ld(gg + k * S, cell));
            }
        }
        collide<R, TH>(h, g, a.col);
#pragma unroll
        for (int q = 0; q < Q19; ++q)
            if (!solid || !((m >> q) & 1u)) st(f + q * S, cell + nb.at(cx19(q), cy19(q), cz19(q)), h[q]);
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k)
                if (!solid || !((m >> k) & 1u)) st(gg + k * S, cell + nb.at(cx7(k), cy7(k), cz7(k)), g[k]);
        }
        if (near) {
#pragma unroll
            for (int q = 1; q < Q19; ++q)
                if ((m >> q) & 1u) st(f + opp19(q) * S, cell, h[q]);
            if (TH) {
#pragma unroll
                for (int k = 1; k < Q7; ++k)
                    if ((m >> k) & 1u) st(gg + opp7(k) * S, cell, solid_rule(a, g[k]));
            }
        }
    }
}

// ------------------------------------------------- two buffers (A-B)

// Collide in place: every population stays in its own slot.
template <typename R, bool TH, bool SOLID>
__global__ void __launch_bounds__(BLOCK) k_ab_collide(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    // solid cells collide NaN in their own slots: nothing else writes this
    // buffer in this kernel and no fluid cell pulls from a solid slot
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

// Pull into the other buffer: B(q, x) = A(q, x - c_q); when x - c_q is a
// solid cell the population comes back from x itself: B(q, x) = A(opp q, x)
// (anti-bounce-back for a Dirichlet D3Q7 population).
template <typename R, bool TH, bool SOLID>
__global__ void __launch_bounds__(BLOCK) k_ab_pull(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    // a solid cell pulls garbage into its own slots of the other buffer, which
    // no fluid cell reads; its mask bits are never those of a fluid cell's
    const uint32_t m = SOLID ? a.mask[cell] : 0u;
    const bool solid = SOLID && (m & MASK_SOLID);
    const int64_t S = G.stride;
    const Nbr nb(G, cell);
#pragma unroll
    for (int q = 0; q < Q19; ++q) {
        R v = ld(a.f + q * S, cell + nb.at(-cx19(q), -cy19(q), -cz19(q)));
        if (SOLID && !solid && ((m >> opp19(q)) & 1u)) v = ld(a.f + opp19(q) * S, cell);
        st(a.f2 + q * S, cell, v);
    }
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) {
            R v = ld(a.g + k * S, cell + nb.at(-cx7(k), -cy7(k), -cz7(k)));
            if (SOLID && !solid && ((m >> opp7(k)) & 1u)) v = solid_rule(a, ld(a.g + opp7(k) * S, cell));
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
// the bounced population f_p^+ of each link where the step left it: for a
// wall link its scatter destination; for a solid link (opp p, x) in place
// (the even step's usual store, or the odd step's bounce-back store) and
// B(opp p, x) with two buffers.  Values a D3Q7 Dirichlet link stores after
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
            if (grp < 6 || a.mode == LINK_AB) {
                const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
                plane = sl.dst_plane;
                idx = sl.dst_idx;
                transformed = true;
            } else {
                plane = opp_rt(p);
                idx = a.cell[l];
                transformed = a.mode == LINK_AA_AFTER_ODD;
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

template <typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_read(FieldArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    const int32_t n = G.ncell;
    R h[Q19];
    R g[Q7];
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
        // an inflow from a solid neighbour is the bounce of the cell's own
        // even-step output, kept in (q, x) (see k_aa_step)
        const uint32_t mk = a.mask ? a.mask[cell] : 0u;
        if (mk != 0 && !(mk & MASK_SOLID)) {
#pragma unroll
            for (int q = 1; q < Q19; ++q)
                if ((mk >> opp19(q)) & 1u) h[q] = a.f[q * S + cell];
            if (TH) {
#pragma unroll
                for (int k = 1; k < Q7; ++k)
                    if ((mk >> opp7(k)) & 1u) {
                        const R v = a.g[k * S + cell];
                        g[k] = a.solid_dirichlet ? a.solid_gw - v : v;
                    }
            }
        }
    }
    Macro<R> m;
    if (a.mask && (a.mask[cell] & MASK_SOLID)) {
        const R nan = (R)__builtin_nan("");
        m.rho = m.ux = m.uy = m.uz = m.T = nan;
    } else {
        m = macros<R, TH>(h, g, a.col);
        const bool bad = !(__builtin_isfinite(m.rho) && __builtin_isfinite(m.T) && __builtin_isfinite(m.ux) &&
                           __builtin_isfinite(m.uy) && __builtin_isfinite(m.uz));
        if (bad) atomicOr(a.unstable, 1);
    }
    if (a.rho_out) a.rho_out[cell] = m.rho;
    if (a.u_out) {
        a.u_out[cell] = m.ux;
        a.u_out[n + cell] = m.uy;
        a.u_out[2 * n + cell] = m.uz;
    }
    if (TH && a.T_out) a.T_out[cell] = m.T;
}

__global__ void __launch_bounds__(BLOCK) k_zero_f64(double* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (i < n) p[i] = 0.0;
}

inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + BLOCK - 1) / BLOCK)); }

}  // namespace

// Pick the <thermal, solid> instance of a cell kernel.
#define LBM_CELL_LAUNCH(KERNEL, a, thermal, s)                                                              \
    do {                                                                                                    \
        const dim3 grid_ = grid_for((a).geo.ncell);                                                         \
        const bool solid_ = (a).mask != nullptr;                                                            \
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
    template hipError_t launch_read<R>(const FieldArgs<R>&, bool, hipStream_t);

LBM_INSTANTIATE(float)
LBM_INSTANTIATE(double)

}  // namespace lbm
