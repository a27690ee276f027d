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

#include "lbm_internal.hpp"

namespace lbm {

namespace {

constexpr int BLOCK = 256;

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

template <typename R, bool TH>
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
        const Nbr nb(G, cell);
#pragma unroll
        for (int q = 0; q < Q19; ++q) h[q] = ld(f + opp19(q) * S, cell + nb.at(-cx19(q), -cy19(q), -cz19(q)));
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) g[k] = ld(gg + opp7(k) * S, cell + nb.at(-cx7(k), -cy7(k), -cz7(k)));
        }
        collide<R, TH>(h, g, a.col);
#pragma unroll
        for (int q = 0; q < Q19; ++q) st(f + q * S, cell + nb.at(cx19(q), cy19(q), cz19(q)), h[q]);
        if (TH) {
#pragma unroll
            for (int k = 0; k < Q7; ++k) st(gg + k * S, cell + nb.at(cx7(k), cy7(k), cz7(k)), g[k]);
        }
    }
}

// ------------------------------------------------- two buffers (A-B)

// Collide in place: every population stays in its own slot.
template <typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_ab_collide(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    R h[Q19];
    R g[Q7];
#pragma unroll
    for (int q = 0; q < Q19; ++q) h[q] = a.f[q * S + cell];
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) g[k] = a.g[k * S + cell];
    }
    collide<R, TH>(h, g, a.col);
#pragma unroll
    for (int q = 0; q < Q19; ++q) a.f[q * S + cell] = h[q];
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) a.g[k * S + cell] = g[k];
    }
}

// Pull into the other buffer: B(q, x) = A(q, x - c_q).
template <typename R, bool TH>
__global__ void __launch_bounds__(BLOCK) k_ab_pull(StepArgs<R> a)
{
    const Geometry& G = a.geo;
    const int32_t cell = (int32_t)(blockIdx.x * BLOCK + threadIdx.x);
    if (cell >= G.ncell) return;
    const int64_t S = G.stride;
    const Nbr nb(G, cell);
#pragma unroll
    for (int q = 0; q < Q19; ++q) a.f2[q * S + cell] = a.f[q * S + (cell + nb.at(-cx19(q), -cy19(q), -cz19(q)))];
    if (TH) {
#pragma unroll
        for (int k = 0; k < Q7; ++k) a.g2[k * S + cell] = a.g[k * S + (cell + nb.at(-cx7(k), -cy7(k), -cz7(k)))];
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

// Reduce the per-lane sums of one wavefront into the group accumulators: a
// wavefront whose links share one group (links are sorted by group) sums with
// shuffles and issues one fp64 atomic per component; a mixed wavefront adds
// lane by lane.  grp < 0 marks lanes without a link.
__device__ __forceinline__ void reduce_to_groups(double* accum, int32_t grp, LinkSum c)
{
    const int32_t lead = __shfl(grp, 0, 64);
    const bool uniform = __all(grp == lead || grp < 0);
    if (uniform) {
        c.fx = wave_sum(c.fx);
        c.fy = wave_sum(c.fy);
        c.fz = wave_sum(c.fz);
        c.q = wave_sum(c.q);
        if ((threadIdx.x & 63) == 0 && lead >= 0) {
            double* acc = accum + 4 * lead;
            atomicAdd(acc + 0, c.fx);
            atomicAdd(acc + 1, c.fy);
            atomicAdd(acc + 2, c.fz);
            atomicAdd(acc + 3, c.q);
        }
    } else if (grp >= 0) {
        double* acc = accum + 4 * grp;
        atomicAdd(acc + 0, c.fx);
        atomicAdd(acc + 1, c.fy);
        atomicAdd(acc + 2, c.fz);
        atomicAdd(acc + 3, c.q);
    }
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
// face, so the two passes keep every source intact.  On a submission's last
// step the gather also takes the momentum exchange and heat.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_gather(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    const int64_t S = a.geo.stride;
    LinkSum c{0.0, 0.0, 0.0, 0.0};
    int32_t grp = -1;
    if (l < a.end) {
        const uint32_t meta = a.meta[l];
        const int p = (int)(meta & LINK_DIR_MASK);
        grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
        const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
        const R* src = (meta & LINK_D3Q7) ? a.g_src : a.f_src;
        const R v = ld(src + sl.src_plane * S, sl.src_idx);
        a.scratch[l] = v;
        if (a.accumulate) c = link_sum(a, meta, p, grp, v);
    }
    if (a.accumulate) reduce_to_groups(a.accum, grp, c);
}

// Scatter (wall links): write each gathered value where the next step reads it.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_scatter(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.end) return;
    const int64_t S = a.geo.stride;
    const uint32_t meta = a.meta[l];
    const int p = (int)(meta & LINK_DIR_MASK);
    const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
    const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
    R* dst = (meta & LINK_D3Q7) ? a.g_dst : a.f_dst;
    st(dst + sl.dst_plane * S, sl.dst_idx, link_value(a, meta, grp, a.scratch[l]));
}

// Direct pass (solid links, and every link with two buffers): gather and
// scatter in one pass.  A solid link's destination is a solid cell's slot
// (after an even step) or a slot of its own fluid cell that only the solid
// neighbour would read (after an odd step); neither is ever another link's
// source, so no scratch is needed.  With two buffers sources and
// destinations lie in different buffers.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_direct(LinkArgs<R> a)
{
    const int64_t l = a.begin + (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    const int64_t S = a.geo.stride;
    LinkSum c{0.0, 0.0, 0.0, 0.0};
    int32_t grp = -1;
    if (l < a.end) {
        const uint32_t meta = a.meta[l];
        const int p = (int)(meta & LINK_DIR_MASK);
        grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
        const LinkSlots sl = link_slots(a.mode, p, a.cell[l], a.cellw[l]);
        const bool g7 = (meta & LINK_D3Q7) != 0;
        const R v = ld((g7 ? a.g_src : a.f_src) + sl.src_plane * S, sl.src_idx);
        st((g7 ? a.g_dst : a.f_dst) + sl.dst_plane * S, sl.dst_idx, link_value(a, meta, grp, v));
        if (a.accumulate) c = link_sum(a, meta, p, grp, v);
    }
    if (a.accumulate) reduce_to_groups(a.accum, grp, c);
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
    if (a.labels && a.labels[cell]) {
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
    }
    Macro<R> m;
    if (a.labels && a.labels[cell]) {
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

template <typename R>
hipError_t launch_aa_step(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_aa_step<R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_aa_step<R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_ab_collide(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_ab_collide<R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_ab_collide<R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_ab_pull(const StepArgs<R>& a, bool thermal, hipStream_t s)
{
    if (thermal) hipLaunchKernelGGL((k_ab_pull<R, true>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_ab_pull<R, false>), grid_for(a.geo.ncell), dim3(BLOCK), 0, s, a);
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
    template hipError_t launch_init<R>(const FieldArgs<R>&, bool, hipStream_t);          \
    template hipError_t launch_read<R>(const FieldArgs<R>&, bool, hipStream_t);

LBM_INSTANTIATE(float)
LBM_INSTANTIATE(double)

}  // namespace lbm
