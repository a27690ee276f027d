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

// Gather: read every link's post-collision source into scratch.  On a
// submission's last step, also sum the momentum exchange 2 c_p f_p^+ (D3Q19
// links) and the heat w T_w - 2 g_p^+ (Dirichlet D3Q7 links) per group: a
// wavefront whose links share one group reduces with shuffles and issues one
// fp64 atomic per component; a mixed wavefront adds lane by lane.
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_gather(LinkArgs<R> a)
{
    const int64_t l = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    const int64_t S = a.geo.stride;
    double fx = 0.0, fy = 0.0, fz = 0.0, qh = 0.0;
    int32_t grp = -1;
    if (l < a.n_total) {
        const bool isf = l < a.n_f;
        const uint32_t meta = a.meta[l];
        const int p = (int)(meta & LINK_DIR_MASK);
        grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
        int32_t plane, idx;
        if (a.mode == LINK_AA_AFTER_EVEN) {
            plane = opp_rt(p);
            idx = a.cell[l];
        } else if (a.mode == LINK_AA_AFTER_ODD) {
            plane = p;
            idx = a.cellw[l];
        } else {
            plane = p;
            idx = a.cell[l];
        }
        const R* src = isf ? a.f_src : a.g_src;
        const R v = src[plane * S + idx];
        a.scratch[l] = v;
        if (a.accumulate) {
            if (isf) {
                const double fv = 2.0 * ((double)v + w19_rt(p));  // stored value is f - w
                fx = dir_comp(CX19, p) * fv;
                fy = dir_comp(CY19, p) * fv;
                fz = dir_comp(CZ19, p) * fv;
            } else if (meta & LINK_DIRICHLET) {
                qh = a.omega * a.wall_T[grp] - 2.0 * (double)v;
            }
        }
    }
    if (!a.accumulate) return;
    const int32_t lead = __shfl(grp, 0, 64);
    const bool uniform = __all(grp == lead || grp < 0);
    if (uniform) {
        fx = wave_sum(fx);
        fy = wave_sum(fy);
        fz = wave_sum(fz);
        qh = wave_sum(qh);
        if ((threadIdx.x & 63) == 0 && lead >= 0) {
            double* acc = a.accum + 4 * lead;
            atomicAdd(acc + 0, fx);
            atomicAdd(acc + 1, fy);
            atomicAdd(acc + 2, fz);
            atomicAdd(acc + 3, qh);
        }
    } else if (grp >= 0) {
        double* acc = a.accum + 4 * grp;
        atomicAdd(acc + 0, fx);
        atomicAdd(acc + 1, fy);
        atomicAdd(acc + 2, fz);
        atomicAdd(acc + 3, qh);
    }
}

// Scatter: write each gathered value where the next step reads it --
// bounce-back f_pbar = f_p^+ (no-slip), anti-bounce-back
// g_pbar = -g_p^+ + w T_w (Dirichlet T), bounce-back g_pbar = g_p^+ (adiabatic).
template <typename R>
__global__ void __launch_bounds__(BLOCK) k_link_scatter(LinkArgs<R> a)
{
    const int64_t l = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
    if (l >= a.n_total) return;
    const int64_t S = a.geo.stride;
    const bool isf = l < a.n_f;
    const uint32_t meta = a.meta[l];
    const int p = (int)(meta & LINK_DIR_MASK);
    R v = a.scratch[l];
    if (!isf && (meta & LINK_DIRICHLET)) {
        const int32_t grp = (int32_t)((meta >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
        v = (R)(a.omega * a.wall_T[grp]) - v;
    }
    int32_t plane, idx;
    if (a.mode == LINK_AA_AFTER_EVEN) {
        plane = p;
        idx = a.cellw[l];
    } else {
        plane = opp_rt(p);
        idx = a.cell[l];
    }
    R* dst = isf ? a.f_dst : a.g_dst;
    dst[plane * S + idx] = v;
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
    if (a.n_total == 0) return hipSuccess;
    hipLaunchKernelGGL((k_link_gather<R>), grid_for(a.n_total), dim3(BLOCK), 0, s, a);
    return hipGetLastError();
}

template <typename R>
hipError_t launch_link_scatter(const LinkArgs<R>& a, hipStream_t s)
{
    if (a.n_total == 0) return hipSuccess;
    hipLaunchKernelGGL((k_link_scatter<R>), grid_for(a.n_total), dim3(BLOCK), 0, s, a);
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
    template hipError_t launch_init<R>(const FieldArgs<R>&, bool, hipStream_t);          \
    template hipError_t launch_read<R>(const FieldArgs<R>&, bool, hipStream_t);

LBM_INSTANTIATE(float)
LBM_INSTANTIATE(double)

}  // namespace lbm
