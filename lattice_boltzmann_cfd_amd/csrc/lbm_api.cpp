// lbm_api.cpp -- the C ABI of include/lbm.h: parameter checks, the host link
// builder, carving of the caller's device buffer and the per-step launch
// sequence.  All arithmetic of the method runs in lbm_kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <iterator>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <thread>
#include <vector>

#include "lbm.h"
#include "lbm_internal.hpp"

using namespace lbm;

struct lbm_ctx {
    lbm_params p;
    int es = 4;
    bool thermal = false;
    bool ab = false;    // two population buffers
    bool push = false;  // ... stepped in one pass (collide and push)
    bool two_d = false;  // D2Q9 + D2Q5 on one z layer
    hipStream_t stream = nullptr;
    int device = 0;  // current device at lbm_create
    Geometry geo{};
    char* f = nullptr;
    char* g = nullptr;
    char* f2 = nullptr;
    char* g2 = nullptr;
    uint32_t* mask = nullptr;
    int32_t* lcell = nullptr;
    int32_t* lcellw = nullptr;
    uint32_t* lmeta = nullptr;
    char* scratch = nullptr;
    char* face_vel = nullptr;  // PRESSURE faces: velocity planes
    double* wall_T = nullptr;
    double* accum = nullptr;
    int64_t* seg_begin = nullptr;  // force-pass segments (see LinkArgs)
    int32_t* group_seg = nullptr;
    double* seg_sum = nullptr;
    int64_t n_seg = 0;
    double* diag = nullptr;
    int32_t* unstable = nullptr;
    int64_t n_f = 0, n_g = 0, n_wall = 0;
    int64_t t = 0;
    bool initialised = false;
    bool in_kernel = false;  // bounce-back inside the step kernel
    size_t lds[2] = {0, 0};  // per parity: local data share reserved per block of the step kernel
    // replay of 8 even+odd pairs of steps as a HIP graph (captured once on a
    // private stream, launched on the caller's)
    hipStream_t capture_stream = nullptr;
    hipGraphExec_t pair = nullptr;
    int pair_steps = 0;  // steps per replay (an even number)
    bool pair_failed = false;
    // per-kernel timing (lbm_profile): an event pair recorded around each
    // launch on the caller's stream, added up at a synchronisation
    struct Timed {
        int kind;
        hipEvent_t start, stop;
    };
    bool profile = false;
    std::vector<Timed> timed;               // recorded, not yet added up
    std::vector<hipEvent_t> spare_events;   // created, free for the next launch
    double prof_ms[LBM_KERNEL_KINDS] = {};
    int64_t prof_launches[LBM_KERNEL_KINDS] = {};
    ~lbm_ctx()
    {
        if (pair) (void)hipGraphExecDestroy(pair);
        if (capture_stream) (void)hipStreamDestroy(capture_stream);
        for (const Timed& t : timed) {
            (void)hipEventDestroy(t.start);
            (void)hipEventDestroy(t.stop);
        }
        for (hipEvent_t e : spare_events) (void)hipEventDestroy(e);
    }
    std::string err;
    Collision<float> colf{};
    Collision<double> cold{};
};

namespace {

thread_local std::string g_create_error;

constexpr size_t ALIGN = 256;
constexpr int64_t MAX_CELLS = (int64_t(1) << 31) - (int64_t(1) << 20);

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

DivMagic make_magic(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t num = uint64_t(1) << (31 + l);
    DivMagic m;
    m.mul = (num + d - 1) / d;
    m.shift = 31 + l;
    m.d = d;
    return m;
}

bool magic_ok(const DivMagic& m, uint32_t limit)
{
    const uint32_t d = m.d;
    const uint32_t probes[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, limit - 1, limit - d, limit / 2,
                               (limit / d) * d, (limit / d) * d - 1, 0x7fffffffu, 0x7ffffffeu};
    for (uint32_t n : probes) {
        if (n > 0x7fffffffu) continue;
        if (divide(n, m) != n / d) return false;
    }
    for (uint32_t n = 0; n < 100000; ++n)
        if (divide(n * 2654435761u % 0x7fffffffu, m) != (n * 2654435761u % 0x7fffffffu) / d) return false;
    return true;
}

bool finite(double v) { return std::isfinite(v); }

// Elements between consecutive population planes: the cell count rounded up
// to a wavefront, plus 1024.  With a power-of-two cell count the planes would
// otherwise start at addresses that agree in every low bit, and the 19 (26)
// accesses of one cell would meet in the same HBM channels and banks.  The
// shift was chosen by measurement on MI355X: in fp32, 1-2 % faster steps at
// 256^3 and 4-8 % at 512^3; in fp64 no change (a 512-element shift is 10-20 %
// slower in either precision, so the value is not arbitrary).
int64_t plane_stride(int64_t n) { return (n + 63) / 64 * 64 + 1024; }

// Words of the mask array before its bitmap (the cell count rounded up to a
// wavefront, so the bitmap starts on a 256-byte boundary).
int64_t mask_words(int64_t n) { return (n + 63) / 64 * 64; }

// One bit per cell, set where the cell's mask word is not 0.
std::vector<uint32_t> near_bits(const std::vector<uint32_t>& mask)
{
    std::vector<uint32_t> bits((mask.size() + 31) / 32, 0u);
    for (size_t i = 0; i < mask.size(); ++i)
        if (mask[i]) bits[i >> 5] |= 1u << (i & 31);
    return bits;
}

// Automatic tiling (lbm_params.tile_log2 = 0): tiles hold 32 KiB of each
// plane (2^13 fp32 or 2^12 fp64 cells), 64 KiB (2^14 fp32 or 2^13 fp64
// cells) for an isothermal fp32 D3Q19 box and a thermal fp64 D3Q19 + D3Q7
// box; a thermal box keeps its temperature planes in the same tiles as its
// flow planes, except the fp64 2D one.  Measured on MI355X in same-box A/B
// runs of this library against one plane per population: 256^3 fp32 step
// -6.1 %, 256^3 thermal fp32 -5.1 % (-1.2 % more with shared tiles), the
// 8193^2 2D cell in fp32 -9.3 % (-2.0 % more), 256^3 fp64 -2.8 % with 2^12
// instead of 2^13 cells; shared tiles cost the fp64 2D cell 6.1 %.  With
// the occupancy bounds, 2^14 instead of 2^13 cells: 256^3 isothermal fp32
// -1.4 % (a sphere in that box and the open channel: within 0.4 %).  The
// thermal fp64 3D kernel in shared tiles of 2^13 cells against its earlier
// layout (separate tiles of 2^12 cells below 4 GiB, one plane per population
// above): 256^3 -0.4 %, 385^3 -8.0 %, 450^3 -8.2 %, 512^3 +1.1 % (with random
// spheres +4.4 %); 2^12 and 2^14 cells were 2.2 % and 1.6 % slower at 385^3.
// Every other instance as fast or faster at 32 KiB per plane.
constexpr int64_t TILE_PLANE_BYTES = 32768;

int64_t tile_plane_bytes(const lbm_params* p)
{
    const bool three_d = p->lattice == LBM_LATTICE_3D;
    const bool iso3d_fp32 = three_d && !p->thermal && p->dtype == 4;
    const bool thermal3d_fp64 = three_d && p->thermal && p->dtype == 8;
    return iso3d_fp32 || thermal3d_fp64 ? 2 * TILE_PLANE_BYTES : TILE_PLANE_BYTES;
}

// Automatic layout of a population buffer of 4 GiB or more: tiles (lane
// offsets of 32-bit elements, scaled to bytes in 64-bit arithmetic) for the
// kernel instances that ran faster that way on MI355X, one plane per
// population for the others.  Same-box A/B of the step: the 512^3 box with
// random spheres (D3Q19 + D3Q7, fp32) -3.5 % tiled (even step -9.8 %), the
// 8193^2 heated cell (D2Q9 + D2Q5, fp64) -4.4 %, heated cavities in fp64
// (D3Q19 + D3Q7) -8 % at 385^3 and 450^3 (+1.1 % at 512^3, +4.4 % for the
// 512^3 random-sphere box: boxes of a power of two suit the planes' shift);
// the periodic box (D3Q19) +1.2 % tiled in fp32 at 512^3 (+4.6 % at 400^3,
// +0.8 % at 450^3, +2.1 % at 480^3) and +5.4 % in fp64 at 512^3 (+2.1 % at
// 448^3, but -6.5 % at 385^3).
bool tiles_for_large_buffers(const lbm_params* p)
{
    const bool two_d = p->lattice == LBM_LATTICE_2D;
    return p->thermal && (!two_d || p->dtype == 8);
}

// Tile geometry of the population buffers (see Geometry).  Tiles are used
// when asked for (tile_log2 in 6..20) or, automatically, when the box holds
// at least four of them and the buffer stays below 4 GiB (or, larger, for the
// instances tiles_for_large_buffers() names); always only while every
// population buffer holds fewer than 2^32 elements, so that a lane's element
// offset from its plane's base fits in 32 bits.  Otherwise one plane per
// population over the whole box (each plane < 4 GiB, checked by validate()).
// Splitting larger buffers into groups of planes that each stay below 4 GiB
// measured slower on MI355X (512^3 thermal 1 %, the 8193^2 fp64 2D cell 5 %)
// than one plane per population.  Writes the element counts of the flow and
// temperature buffers and, when the temperature planes share the flow
// planes' tiles, the element offset of the temperature buffer inside the flow
// buffer (else -1).
void tile_geometry(const lbm_params* p, Geometry* G, int64_t* elems_f, int64_t* elems_g, int64_t* g_in_f)
{
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    const bool two_d = p->lattice == LBM_LATTICE_2D;
    const int64_t Q = two_d ? Q9 : Q19, QT = two_d ? Q5 : Q7;
    const bool automatic = p->tile_log2 == 0;
    uint32_t lg = (uint32_t)p->tile_log2;
    if (automatic) {
        lg = 0;
        while ((int64_t(1) << (lg + 1)) * p->dtype <= tile_plane_bytes(p)) ++lg;
    }
    *g_in_f = -1;
    if (lg < 31 && (!automatic || n >= (int64_t(4) << lg))) {
        const int64_t A = int64_t(1) << lg;
        const int64_t tiles = (n + A - 1) >> lg;
        const int64_t limit = (int64_t(1) << 32) - (int64_t(1) << 20);
        const bool shared = p->thermal && (automatic ? p->dtype == 4 || !two_d : true);
        const int64_t QF = shared ? Q + QT : Q;
        const bool small = tiles * QF * A * p->dtype < limit;
        const bool allowed = small || !automatic || tiles_for_large_buffers(p);
        if (QF * A < (int64_t(1) << 24) && tiles * QF * A < limit && allowed) {
            G->tile_lg = lg;
            G->tile_mask = (uint32_t)(A - 1);
            G->qstride = A;
            G->tile_f = (uint32_t)(QF * A);
            G->tile_g = (uint32_t)(shared ? QF * A : QT * A);
            *elems_f = tiles * QF * A;
            *elems_g = shared ? 0 : tiles * QT * A;
            if (shared) *g_in_f = Q * A;
            return;
        }
    }
    const int64_t S = plane_stride(n);
    G->tile_lg = 31;
    G->tile_mask = 0x7fffffffu;
    G->qstride = S;
    G->tile_f = G->tile_g = 0;
    *elems_f = Q * S;
    *elems_g = QT * S;
}

inline bool nonperiodic(const lbm_params* p, int f) { return p->face_kind[f] != LBM_FACE_PERIODIC; }

// A solid cell in the first cell layer of a SLIP face (not supported: the
// reflected populations travel along that layer).
bool solid_on_slip_layer(const lbm_params* p, const uint8_t* labels)
{
    if (!labels) return false;
    const int n[3] = {p->nx, p->ny, p->nz};
    for (int f = 0; f < 6; ++f) {
        if (p->face_kind[f] != LBM_FACE_SLIP) continue;
        const int a = f / 2, b = (a + 1) % 3, d = (a + 2) % 3;  // the face's normal axis and its two in-plane axes
        int c[3];
        c[a] = (f & 1) ? n[a] - 1 : 0;
        for (c[d] = 0; c[d] < n[d]; ++c[d])
            for (c[b] = 0; c[b] < n[b]; ++c[b])
                if (labels[c[0] + (int64_t)n[0] * (c[1] + (int64_t)n[1] * c[2])]) return true;
    }
    return false;
}

// Returns an empty string when the parameters are acceptable.
std::string validate(const lbm_params* p)
{
    if (!p) return "params is NULL";
    if (p->nx < 1 || p->ny < 1 || p->nz < 1) return "nx, ny, nz must be >= 1";
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    if (n >= MAX_CELLS) return "nx*ny*nz too large for 32-bit cell indices";
    if (p->dtype != 4 && p->dtype != 8) return "dtype must be 4 or 8";
    // kernels address a population plane with 32-bit byte offsets
    if (plane_stride(n) * (int64_t)p->dtype >= (int64_t(1) << 32) - (int64_t(1) << 20))
        return "nx*ny*nz*dtype too large for 32-bit plane offsets";
    if (p->streaming < 0 || p->streaming > 3) return "streaming must be 0, 1, 2 or 3";
    if (p->thermal != 0 && p->thermal != 1) return "thermal must be 0 or 1";
    if (p->links != LBM_LINKS_IN_KERNEL && p->links != LBM_LINKS_PASSES) return "links must be 0 or 1";
    bool open = false;
    for (int f = 0; f < 6; ++f) {
        const int k = p->face_kind[f];
        if (k < LBM_FACE_PERIODIC || k > LBM_FACE_PRESSURE) return "bad face_kind";
        if (p->face_thermal[f] != LBM_ADIABATIC && p->face_thermal[f] != LBM_DIRICHLET) return "bad face_thermal";
        if (!finite(p->face_T[f])) return "face_T must be finite";
        for (int a = 0; a < 3; ++a)
            if (!finite(p->face_u[f][a])) return "face_u must be finite";
        if ((k == LBM_FACE_VELOCITY || k == LBM_FACE_PRESSURE) && !(finite(p->face_rho[f]) && p->face_rho[f] > 0.0))
            return "face_rho of a VELOCITY or PRESSURE face must be finite and > 0";
        open = open || k > LBM_FACE_WALL;
    }
    for (int a = 0; a < 3; ++a)
        if ((p->face_kind[2 * a] == LBM_FACE_PERIODIC) != (p->face_kind[2 * a + 1] == LBM_FACE_PERIODIC))
            return "the two faces of an axis must both be periodic or both be non-periodic";
    if (open && p->links != LBM_LINKS_IN_KERNEL)
        return "SLIP, VELOCITY and PRESSURE faces need links = LBM_LINKS_IN_KERNEL";
    if (p->streaming == LBM_STREAM_AB_PUSH && p->links != LBM_LINKS_IN_KERNEL)
        return "streaming = LBM_STREAM_AB_PUSH needs links = LBM_LINKS_IN_KERNEL";
    if (p->solid_thermal != LBM_ADIABATIC && p->solid_thermal != LBM_DIRICHLET) return "bad solid_thermal";
    if (!finite(p->solid_T)) return "solid_T must be finite";
    if (p->lattice != LBM_LATTICE_3D && p->lattice != LBM_LATTICE_2D) return "lattice must be 0 (3D) or 1 (2D)";
    if (!(p->tile_log2 == 0 || p->tile_log2 == 31 || (p->tile_log2 >= 6 && p->tile_log2 <= 20)))
        return "tile_log2 must be 0 (automatic), 6..20 or 31 (no tiles)";
    for (int k = 0; k < 2; ++k)
        if (p->occupancy[k] < -1 || p->occupancy[k] > 8)
            return "occupancy values must be -1 (no bound), 0 (automatic) or 1..8 blocks per compute unit";
    if (p->lattice == LBM_LATTICE_3D) {
        for (int k = 0; k < 19; ++k)
            if (!(p->s19[k] >= 0.0 && p->s19[k] < 2.0)) return "s19 rates must lie in [0, 2)";
        for (int k = 0; k < 7; ++k)
            if (!(p->s7[k] >= 0.0 && p->s7[k] < 2.0)) return "s7 rates must lie in [0, 2)";
        if (!(p->a_T > -6.0 && p->a_T <= 1.0)) return "a_T must lie in (-6, 1]";
    } else {
        if (p->nz != 1) return "a 2D box (D2Q9 + D2Q5) needs nz = 1";
        if (p->face_kind[4] != LBM_FACE_PERIODIC || p->face_kind[5] != LBM_FACE_PERIODIC)
            return "a 2D box needs periodic z faces";
        for (int k = 0; k < 9; ++k)
            if (!(p->s9[k] >= 0.0 && p->s9[k] < 2.0)) return "s9 rates must lie in [0, 2)";
        for (int k = 0; k < 5; ++k)
            if (!(p->s5[k] >= 0.0 && p->s5[k] < 2.0)) return "s5 rates must lie in [0, 2)";
        if (!(p->a_T > -4.0 && p->a_T <= 1.0)) return "a_T must lie in (-4, 1] for D2Q5";
        if (p->accel[2] != 0.0 || p->gbeta[2] != 0.0) return "accel[2] and gbeta[2] must be 0 in 2D";
        for (int f = 0; f < 6; ++f)
            if (p->face_u[f][2] != 0.0) return "face_u z components must be 0 in 2D";
    }
    for (int a = 0; a < 3; ++a)
        if (!finite(p->accel[a]) || !finite(p->gbeta[a])) return "accel and gbeta must be finite";
    if (!finite(p->T0)) return "T0 must be finite";
    return "";
}

template <typename R>
Collision<R> make_collision(const lbm_params* p)
{
    Collision<R> c{};
    const double* s = p->s19;
    c.s_e = (R)s[1];
    c.s_eps = (R)s[2];
    c.s_qx = (R)s[4];
    c.s_qy = (R)s[6];
    c.s_qz = (R)s[8];
    c.s_3pxx = (R)s[9];
    c.s_3pixx = (R)s[10];
    c.s_pww = (R)s[11];
    c.s_piww = (R)s[12];
    c.s_pxy = (R)s[13];
    c.s_pyz = (R)s[14];
    c.s_pxz = (R)s[15];
    c.s_mx = (R)s[16];
    c.s_my = (R)s[17];
    c.s_mz = (R)s[18];
    c.q_jx = (R)p->s7[1];
    c.q_jy = (R)p->s7[2];
    c.q_jz = (R)p->s7[3];
    c.q_e = (R)p->s7[4];
    c.q_5 = (R)p->s7[5];
    c.q_6 = (R)p->s7[6];
    for (int a = 0; a < 3; ++a) {
        c.accel[a] = (R)p->accel[a];
        c.gbeta[a] = p->thermal ? (R)p->gbeta[a] : R(0);
    }
    c.T0 = (R)p->T0;
    c.a_T = (R)p->a_T;
    const double* s2 = p->s9;
    c.s2_e = (R)s2[1];
    c.s2_eps = (R)s2[2];
    c.s2_qx = (R)s2[4];
    c.s2_qy = (R)s2[6];
    c.s2_pxx = (R)s2[7];
    c.s2_pxy = (R)s2[8];
    c.q2_jx = (R)p->s5[1];
    c.q2_jy = (R)p->s5[2];
    c.q2_e = (R)p->s5[3];
    c.q2_4 = (R)p->s5[4];
    return c;
}

// Anti-bounce-back constant of the temperature lattice ("Multi-GPU thermal
// lattice Boltzmann simulations using OpenACC and MPI", Sec. 2):
// (6 + a_T)/21 for D3Q7, (4 + a_T)/10 for D2Q5.
double abb_omega(const lbm_params* p)
{
    return p->lattice == LBM_LATTICE_2D ? (4.0 + p->a_T) / 10.0 : (6.0 + p->a_T) / 21.0;
}

// Velocities of the flow (temp = false) or temperature lattice, rest excluded.
int lattice_dirs(const lbm_params* p, bool temp, int (*c)[3])
{
    int n = 0;
    if (p->lattice == LBM_LATTICE_2D) {
        if (!temp)
            for (int q = 1; q < Q9; ++q) c[n][0] = cx9(q), c[n][1] = cy9(q), c[n][2] = 0, ++n;
        else
            for (int k = 1; k < Q5; ++k) c[n][0] = cx7(k), c[n][1] = cy7(k), c[n][2] = 0, ++n;
    } else {
        if (!temp)
            for (int q = 1; q < Q19; ++q) c[n][0] = cx19(q), c[n][1] = cy19(q), c[n][2] = cz19(q), ++n;
        else
            for (int k = 1; k < Q7; ++k) c[n][0] = cx7(k), c[n][1] = cy7(k), c[n][2] = cz7(k), ++n;
    }
    return n;
}

// Cells of face f (x faces: ny*nz, y faces: nx*nz, z faces: nx*ny).
int64_t face_area(const lbm_params* p, int f)
{
    const int a = f / 2;
    return a == 0 ? (int64_t)p->ny * p->nz : (a == 1 ? (int64_t)p->nx * p->nz : (int64_t)p->nx * p->ny);
}

// Element offsets of the PRESSURE faces' velocity planes (3 planes of the
// face's area each); returns the total element count.
int64_t face_planes(const lbm_params* p, int64_t* off)
{
    int64_t total = 0;
    for (int f = 0; f < 6; ++f) {
        off[f] = -1;
        if (p->face_kind[f] != LBM_FACE_PRESSURE) continue;
        off[f] = total;
        total += 3 * face_area(p, f);
    }
    return total;
}

template <typename R>
Bounce<R> make_bounce(const lbm_params* p, bool in_kernel, void* face_vel)
{
    Bounce<R> b{};
    const double omega = abb_omega(p);
    for (int f = 0; f < 6; ++f) {
        b.face_gw[f] = (R)(omega * p->face_T[f]);
        if (nonperiodic(p, f)) b.walls |= 1 << f;
        if (p->face_kind[f] == LBM_FACE_SLIP) b.slip |= 1 << f;
        if (p->face_kind[f] == LBM_FACE_VELOCITY) b.vel |= 1 << f;
        if (p->face_kind[f] == LBM_FACE_PRESSURE) b.pres |= 1 << f;
        if (p->face_thermal[f] == LBM_DIRICHLET) b.face_dirichlet |= 1 << f;
        b.face_rho[f] = (R)p->face_rho[f];
        for (int a = 0; a < 3; ++a) b.face_u[f][a] = (R)p->face_u[f][a];
        b.face_area[f] = face_area(p, f);
    }
    face_planes(p, b.face_off);
    b.near_off = (int32_t)mask_words((int64_t)p->nx * p->ny * p->nz);
    b.face_vel = (R*)face_vel;
    b.solid_gw = (R)(omega * p->solid_T);
    b.solid_dirichlet = p->solid_thermal == LBM_DIRICHLET ? 1 : 0;
    b.in_kernel = in_kernel ? 1 : 0;
    return b;
}

// ------------------------------------------------------------- occupancy

// Blocks per compute unit that occupancy = 0 gives the in-place step kernel,
// for the even and the odd step (-1: no bound).  Chosen by interleaved
// timings on MI355X of whole steps at bounds of 1 to 4 blocks and none, on
// 256^3 periodic boxes (D3Q19, fp32 and fp64), a sphere in a 256^3 box (fp32,
// fp64), the heated 256^3 cavity (D3Q19 + D3Q7, fp32 and fp64), a 512^3 box
// with random spheres, 8192^2 periodic and 8193^2 heated squares (D2Q9, and
// with D2Q5, fp32 and fp64) and channels of 256x128x128 and 512x256x256
// cells with a velocity inlet and a pressure outlet (open faces: every bound
// was slower).  Instances not listed keep the bound their registers give.
struct OccupancyChoice {
    int lattice, dtype, thermal, rules, even, odd;
};
constexpr OccupancyChoice OCCUPANCY_TABLE[] = {
    {LBM_LATTICE_3D, 4, 0, 0, 2, 2},
    {LBM_LATTICE_3D, 4, 0, 1, 2, 3},
    {LBM_LATTICE_3D, 4, 1, 1, 2, -1},
    {LBM_LATTICE_3D, 8, 0, 0, 1, 2},
    {LBM_LATTICE_3D, 8, 0, 1, 1, 2},
    {LBM_LATTICE_3D, 8, 1, 1, 1, 2},
    {LBM_LATTICE_2D, 4, 0, 0, 3, 3},
    {LBM_LATTICE_2D, 4, 1, 1, 3, 4},
    {LBM_LATTICE_2D, 8, 0, 0, 2, 2},
    {LBM_LATTICE_2D, 8, 1, 1, 2, 2},
};
// The same for the one-pass two-buffer kernel (LBM_STREAM_AB_PUSH), timed on
// the same boxes at bounds of 1 to 4 blocks and none; open faces again ran
// fastest unbounded.  The two-pass two-buffer kernels keep no bound.
constexpr OccupancyChoice PUSH_OCCUPANCY_TABLE[] = {
    {LBM_LATTICE_3D, 4, 0, 0, 3, 3},
    {LBM_LATTICE_3D, 4, 0, 1, 3, 3},
    {LBM_LATTICE_3D, 4, 1, 1, 2, 2},
    {LBM_LATTICE_3D, 8, 0, 0, 2, 2},
    {LBM_LATTICE_3D, 8, 1, 1, 2, 2},
    {LBM_LATTICE_2D, 4, 0, 0, 3, 3},
    {LBM_LATTICE_2D, 4, 1, 1, 2, 2},
    {LBM_LATTICE_2D, 8, 1, 1, 2, 2},
};

int automatic_occupancy(const lbm_params* p, bool ab, bool push, int rules, int parity)
{
    if (ab && !push) return -1;
    const OccupancyChoice* table = push ? PUSH_OCCUPANCY_TABLE : OCCUPANCY_TABLE;
    const size_t n = push ? std::size(PUSH_OCCUPANCY_TABLE) : std::size(OCCUPANCY_TABLE);
    for (size_t i = 0; i < n; ++i) {
        const OccupancyChoice& o = table[i];
        if (o.lattice == p->lattice && o.dtype == p->dtype && o.thermal == p->thermal && o.rules == rules)
            return parity ? o.odd : o.even;
    }
    return -1;
}

// Bytes of local data share to reserve per block so that at most `blocks`
// blocks fit on a compute unit holding lds_cu bytes (0: no reservation).
// The step kernels use no local data share themselves.
size_t occupancy_lds(int blocks, int lds_cu)
{
    if (blocks < 1 || lds_cu <= 0) return 0;
    const size_t per = (size_t)lds_cu / (size_t)blocks / 1024 * 1024 - 1024;
    if (per == 0 || per * (size_t)blocks > (size_t)lds_cu || per * (size_t)(blocks + 1) <= (size_t)lds_cu) return 0;
    return per;
}

// ------------------------------------------------------------- links

struct LinkList {
    std::vector<int32_t> cell, cellw;
    std::vector<uint32_t> meta;
};

struct Dir {
    int c[3];
};

// For fluid cell (x, y, z) and direction c: the group of the blocked link, or
// -1.  A link is blocked when x + c leaves the box through a non-periodic
// face (the first crossed axis in x, y, z order governs) or its periodic
// image is solid.  *rule and *axis give the face's rule (a link crossing two
// faces bounces back where the first one is SLIP) and the governing axis.
inline int blocked_group(const lbm_params* p, const uint8_t* labels, int x, int y, int z, const int* c,
                         int32_t* image, uint32_t* rule = nullptr, int* axis = nullptr)
{
    const int n[3] = {p->nx, p->ny, p->nz};
    int t[3] = {x + c[0], y + c[1], z + c[2]};
    int grp = -1, crossed = 0;
    for (int a = 0; a < 3; ++a) {
        int f = -1;
        if (t[a] < 0 && nonperiodic(p, 2 * a)) f = 2 * a;
        else if (t[a] >= n[a] && nonperiodic(p, 2 * a + 1)) f = 2 * a + 1;
        if (f < 0) continue;
        ++crossed;
        if (grp < 0) grp = f;
    }
    for (int a = 0; a < 3; ++a) t[a] = t[a] < 0 ? t[a] + n[a] : (t[a] >= n[a] ? t[a] - n[a] : t[a]);
    *image = t[0] + p->nx * (t[1] + p->ny * t[2]);
    if (rule) *rule = RULE_WALL;
    if (axis) *axis = grp >= 0 ? grp / 2 : 0;
    if (grp >= 0) {
        const int k = p->face_kind[grp];
        if (rule) {
            *rule = k == LBM_FACE_SLIP ? (crossed > 1 ? RULE_WALL : RULE_SLIP)
                  : k == LBM_FACE_VELOCITY ? RULE_VELOCITY
                  : k == LBM_FACE_PRESSURE ? RULE_PRESSURE : RULE_WALL;
        }
        return grp;
    }
    if (labels && labels[*image]) return 5 + labels[*image];
    return -1;
}

// Build (or only count) the links of one lattice.  Cells are visited in
// index order by several host threads; the result is then ordered by group
// with a stable counting sort so that wavefronts of the gather pass mostly
// see a single group.
int64_t build_links(const lbm_params* p, const uint8_t* labels, bool temp, LinkList* out)
{
    std::vector<Dir> dirs;
    int c[Q19][3];
    const int nd = lattice_dirs(p, temp, c);
    for (int i = 0; i < nd; ++i) dirs.push_back({{c[i][0], c[i][1], c[i][2]}});
    const int nz = p->nz;
    unsigned nthreads = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    nthreads = std::min<unsigned>(nthreads, (unsigned)nz);
    std::vector<LinkList> parts(nthreads);
    std::vector<int64_t> counts(nthreads, 0);
    const bool walls_x = nonperiodic(p, 0);
    const bool walls_y = nonperiodic(p, 2);
    const bool walls_z = nonperiodic(p, 4);

    auto work = [&](unsigned tid) {
        const int z0 = (int)((int64_t)nz * tid / nthreads), z1 = (int)((int64_t)nz * (tid + 1) / nthreads);
        LinkList& L = parts[tid];
        int64_t cnt = 0;
        for (int z = z0; z < z1; ++z)
            for (int y = 0; y < p->ny; ++y)
                for (int x = 0; x < p->nx; ++x) {
                    const int32_t cell = x + p->nx * (y + p->ny * z);
                    if (labels && labels[cell]) continue;
                    const bool edge = (walls_x && (x == 0 || x == p->nx - 1)) ||
                                      (walls_y && (y == 0 || y == p->ny - 1)) ||
                                      (walls_z && (z == 0 || z == nz - 1));
                    if (!edge && !labels) continue;
                    for (size_t i = 0; i < dirs.size(); ++i) {
                        int32_t image;
                        uint32_t rule;
                        int axis;
                        const int grp = blocked_group(p, labels, x, y, z, dirs[i].c, &image, &rule, &axis);
                        if (grp < 0) continue;
                        ++cnt;
                        if (!out) continue;
                        uint32_t meta = (uint32_t)(i + 1) | ((uint32_t)grp << LINK_GROUP_SHIFT);
                        if (temp) {
                            meta |= LINK_TEMP;
                            const int dir = grp < 6 ? p->face_thermal[grp] : p->solid_thermal;
                            if (dir == LBM_DIRICHLET) meta |= LINK_DIRICHLET;
                        } else {
                            meta |= (rule << LINK_RULE_SHIFT) | ((uint32_t)axis << LINK_AXIS_SHIFT);
                            if (rule == RULE_SLIP) {
                                // the reflected population lands at x + c_t
                                int t[3] = {x, y, z};
                                const int n3[3] = {p->nx, p->ny, p->nz};
                                for (int a = 0; a < 3; ++a) {
                                    if (a != axis) t[a] += dirs[i].c[a];
                                    t[a] = t[a] < 0 ? t[a] + n3[a] : (t[a] >= n3[a] ? t[a] - n3[a] : t[a]);
                                }
                                image = t[0] + p->nx * (t[1] + p->ny * t[2]);
                            } else if (rule == RULE_PRESSURE) {
                                image = axis == 0 ? y + p->ny * z : (axis == 1 ? x + p->nx * z : x + p->nx * y);
                            }
                        }
                        L.cell.push_back(cell);
                        L.cellw.push_back(image);
                        L.meta.push_back(meta);
                    }
                }
        counts[tid] = cnt;
    };
    std::vector<std::thread> pool;
    for (unsigned t = 1; t < nthreads; ++t) pool.emplace_back(work, t);
    work(0);
    for (auto& th : pool) th.join();
    int64_t total = 0;
    for (auto c : counts) total += c;
    if (!out) return total;

    out->cell.reserve(total);
    out->cellw.reserve(total);
    out->meta.reserve(total);
    for (auto& L : parts) {
        out->cell.insert(out->cell.end(), L.cell.begin(), L.cell.end());
        out->cellw.insert(out->cellw.end(), L.cellw.begin(), L.cellw.end());
        out->meta.insert(out->meta.end(), L.meta.begin(), L.meta.end());
    }
    return total;
}

// Order both lattices' links for the passes: a stable counting sort by
// (group, lattice, direction) keeps cell order inside each bucket, so wall
// links (groups 0..5) come first and neighbouring lanes of a wavefront read
// one population plane at nearby cells, and a wavefront rarely spans two
// groups (the force reduction).
int64_t order_links(const LinkList& f, const LinkList& g, LinkList* out)
{
    constexpr int NB = LBM_MAX_GROUPS * 2 * 32;
    auto bucket_of = [](uint32_t m) {
        const uint32_t grp = (m >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK;
        return (int)((grp * 2 + ((m & LINK_TEMP) ? 1 : 0)) * 32 + (m & LINK_DIR_MASK));
    };
    std::vector<int64_t> start(NB + 1, 0);
    for (const LinkList* L : {&f, &g})
        for (uint32_t m : L->meta) ++start[bucket_of(m) + 1];
    for (int b = 0; b < NB; ++b) start[b + 1] += start[b];
    const int64_t total = start[NB];
    out->cell.resize(total);
    out->cellw.resize(total);
    out->meta.resize(total);
    for (const LinkList* L : {&f, &g})
        for (size_t i = 0; i < L->meta.size(); ++i) {
            const int64_t pos = start[bucket_of(L->meta[i])]++;
            out->cell[pos] = L->cell[i];
            out->cellw[pos] = L->cellw[i];
            out->meta[pos] = L->meta[i];
        }
    int64_t n_wall = 0;
    while (n_wall < total && ((out->meta[n_wall] >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK) < 6) ++n_wall;
    return n_wall;
}

bool any_solid(const lbm_params* p, const uint8_t* labels)
{
    if (!labels) return false;
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    for (int64_t i = 0; i < n; ++i)
        if (labels[i]) return true;
    return false;
}

// Per-cell solid mask.  Fluid cell: bit q (flow direction 1..18 or 1..8) when the
// link (x, q) ends in a solid cell without crossing a wall face.  Solid cell:
// MASK_SOLID, and bit q when (s + c_q, opp q) is such a link of a fluid cell.
std::vector<uint32_t> build_mask(const lbm_params* p, const uint8_t* labels)
{
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    std::vector<uint32_t> mask((size_t)n, 0u);
    const int nz = p->nz;
    int dirs[Q19][3];
    const int nd = lattice_dirs(p, false, dirs);
    unsigned nthreads = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    nthreads = std::min<unsigned>(nthreads, (unsigned)nz);
    auto work = [&](unsigned tid) {
        const int z0 = (int)((int64_t)nz * tid / nthreads), z1 = (int)((int64_t)nz * (tid + 1) / nthreads);
        for (int z = z0; z < z1; ++z)
            for (int y = 0; y < p->ny; ++y)
                for (int x = 0; x < p->nx; ++x) {
                    const int32_t cell = x + p->nx * (y + p->ny * z);
                    uint32_t m = 0;
                    for (int q = 1; q <= nd; ++q) {
                        const int c[3] = {dirs[q - 1][0], dirs[q - 1][1], dirs[q - 1][2]};
                        int32_t image;
                        if (!labels[cell]) {
                            if (blocked_group(p, labels, x, y, z, c, &image) >= 6) m |= 1u << q;
                            continue;
                        }
                        // solid cell: does the fluid neighbour at s + c_q bounce off s?
                        const int t[3] = {x + c[0], y + c[1], z + c[2]};
                        const int n3[3] = {p->nx, p->ny, p->nz};
                        bool crosses = false;
                        int w[3];
                        for (int a = 0; a < 3; ++a) {
                            if ((t[a] < 0 || t[a] >= n3[a]) && nonperiodic(p, 2 * a)) crosses = true;
                            w[a] = t[a] < 0 ? t[a] + n3[a] : (t[a] >= n3[a] ? t[a] - n3[a] : t[a]);
                        }
                        if (!crosses && !labels[w[0] + p->nx * (w[1] + p->ny * w[2])]) m |= 1u << q;
                    }
                    mask[cell] = labels[cell] ? (m | MASK_SOLID) : m;
                }
    };
    std::vector<std::thread> pool;
    for (unsigned t = 1; t < nthreads; ++t) pool.emplace_back(work, t);
    work(0);
    for (auto& th : pool) th.join();
    return mask;
}

// Run-time check that no two links store into one slot, and that no solid
// cell's odd-step store meets a fluid neighbour's bounce-back store (the
// in-place scheme needs every slot written by exactly one cell per step).
// The stores the link lists stand for:
//  * bounce-back inside the step kernel (odd step, and the one-pass
//    two-buffer step): a link (x, p) stores the returning population at
//    (opp p, x), a SLIP link at (p reflected, x + c_t), a temperature link at
//    (opp k, x);
//  * link passes after an even step: (p, x + c_p) (the link's cellw);
//    after an odd step: (opp p, x).
// A solid cell s stores direction q at (q, s + c_q) unless its mask marks q
// as claimed; a solid link (x, p) with s = x + c_p stores at (opp p, x), so
// s must mark opp p.  The links are bucketed by plane and each plane's cells
// marked in one reusable bitmap of nx*ny*nz bits: O(links) time.  Returns an
// empty string when the links are consistent.
std::string check_link_destinations(const lbm_params* p, const LinkList& L, const std::vector<uint32_t>* mask,
                                    bool passes)
{
    const bool two_d = p->lattice == LBM_LATTICE_2D;
    const int Qf = two_d ? Q9 : Q19, Qt = two_d ? Q5 : Q7;
    int cf[Q19][3], ct[Q7][3];
    lattice_dirs(p, false, cf);
    lattice_dirs(p, true, ct);
    // c[d] of direction d (0 = rest) of either lattice, and its opposite / reflections
    auto comp = [&](bool temp, int d, int a) { return d == 0 ? 0 : (temp ? ct[d - 1][a] : cf[d - 1][a]); };
    auto find = [&](bool temp, int x, int y, int z) {
        const int nq = temp ? Qt : Qf;
        for (int r = 0; r < nq; ++r)
            if (comp(temp, r, 0) == x && comp(temp, r, 1) == y && comp(temp, r, 2) == z) return r;
        return -1;
    };
    // tables: opposite directions of both lattices, reflections across each axis
    int opp_t[2][Q19], refl_t[3][Q19];
    for (int t = 0; t < 2; ++t)
        for (int d = 0; d < (t ? Qt : Qf); ++d)
            opp_t[t][d] = find(t != 0, -comp(t != 0, d, 0), -comp(t != 0, d, 1), -comp(t != 0, d, 2));
    for (int a = 0; a < 3; ++a)
        for (int d = 0; d < Qf; ++d) {
            int c[3] = {comp(false, d, 0), comp(false, d, 1), comp(false, d, 2)};
            c[a] = -c[a];
            refl_t[a][d] = find(false, c[0], c[1], c[2]);
        }
    auto opposite = [&](bool temp, int d) { return opp_t[temp ? 1 : 0][d]; };
    auto reflected = [&](int d, int a) { return refl_t[a][d]; };
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    const int64_t nl = (int64_t)L.meta.size();
    const int planes = Qf + Qt;
    std::vector<int64_t> start(planes + 1);
    std::vector<int32_t> cells(nl);
    std::vector<uint64_t> bits((size_t)((n + 63) / 64), 0u);
    auto check_set = [&](auto slot_of, const char* what) -> std::string {
        // counting sort of the links' destination cells by plane
        std::fill(start.begin(), start.end(), 0);
        for (int64_t l = 0; l < nl; ++l) {
            int32_t cell;
            ++start[slot_of(l, &cell) + 1];
        }
        for (int q = 0; q < planes; ++q) start[q + 1] += start[q];
        std::vector<int64_t> pos(start.begin(), start.end() - 1);
        for (int64_t l = 0; l < nl; ++l) {
            int32_t cell;
            const int q = slot_of(l, &cell);
            cells[pos[q]++] = cell;
        }
        for (int q = 0; q < planes; ++q) {
            std::string err;
            for (int64_t i = start[q]; i < start[q + 1] && err.empty(); ++i) {
                const int32_t c = cells[i];
                uint64_t& w = bits[(size_t)c >> 6];
                const uint64_t b = uint64_t(1) << (c & 63);
                if (w & b) err = std::string("two links store into one slot (") + what + ", plane " +
                                 std::to_string(q) + ", cell " + std::to_string(c) + ")";
                w |= b;
            }
            for (int64_t i = start[q]; i < start[q + 1]; ++i) bits[(size_t)cells[i] >> 6] = 0u;
            if (!err.empty()) return err;
        }
        return "";
    };
    auto unpack = [&](int64_t l, bool* temp, int* d, uint32_t* rule, int* axis) {
        const uint32_t m = L.meta[l];
        *temp = (m & LINK_TEMP) != 0;
        *d = (int)(m & LINK_DIR_MASK);
        *rule = (m >> LINK_RULE_SHIFT) & 3u;
        *axis = (int)((m >> LINK_AXIS_SHIFT) & 3u);
    };
    // bounce-back stores (in the step kernel) and link-pass stores after an odd step
    std::string err = check_set(
        [&](int64_t l, int32_t* cell) {
            bool temp;
            int d, axis;
            uint32_t rule;
            unpack(l, &temp, &d, &rule, &axis);
            if (!temp && rule == RULE_SLIP) {
                *cell = L.cellw[l];
                return reflected(d, axis);
            }
            *cell = L.cell[l];
            return (temp ? Qf : 0) + opposite(temp, d);
        },
        "returning populations");
    if (err.empty() && passes)
        err = check_set(
            [&](int64_t l, int32_t* cell) {
                bool temp;
                int d, axis;
                uint32_t rule;
                unpack(l, &temp, &d, &rule, &axis);
                *cell = L.cellw[l];
                return (temp ? Qf : 0) + d;
            },
            "link passes after an even step");
    if (!err.empty() || !mask || passes) return err;
    for (int64_t l = 0; l < nl; ++l) {
        const uint32_t m = L.meta[l];
        const int grp = (int)((m >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK);
        if (grp < 6 || (m & LINK_TEMP)) continue;
        const int d = (int)(m & LINK_DIR_MASK);
        const uint32_t ms = (*mask)[(size_t)L.cellw[l]];
        const int o = opposite(false, d);
        if (!(ms & MASK_SOLID) || !((ms >> o) & 1u))
            return "solid cell " + std::to_string(L.cellw[l]) + " does not leave direction " + std::to_string(o) +
                   " to the fluid cell " + std::to_string(L.cell[l]) + " that bounces into that slot";
    }
    return "";
}

struct Layout {
    size_t f, g, f2, g2, mask, lcell, lcellw, lmeta, scratch, face_vel, wall_T, accum, seg_begin, group_seg, seg_sum,
        diag, unstable, total;
    Geometry tiles;  // the tile fields of the kernels' Geometry
};

// Force-pass segments: each group's links (contiguous after order_links) cut
// into runs of at most LINK_SEGMENT links.  A group of n links gives
// ceil(n / LINK_SEGMENT) segments, so all groups together give at most
// n_links / LINK_SEGMENT + 1 + LBM_MAX_GROUPS.
size_t max_segments(int64_t n_links) { return (size_t)(n_links / LINK_SEGMENT) + 1 + LBM_MAX_GROUPS; }

void build_segments(const std::vector<uint32_t>& meta, std::vector<int64_t>* seg_begin, std::vector<int32_t>* group_seg)
{
    const int64_t n = (int64_t)meta.size();
    seg_begin->clear();
    group_seg->assign(LBM_MAX_GROUPS + 1, 0);
    int64_t l = 0;
    for (int g = 0; g < LBM_MAX_GROUPS; ++g) {
        (*group_seg)[g] = (int32_t)seg_begin->size();
        int64_t e = l;
        while (e < n && (int)((meta[e] >> LINK_GROUP_SHIFT) & LINK_GROUP_MASK) == g) ++e;
        for (int64_t b = l; b < e; b += LINK_SEGMENT) seg_begin->push_back(b);
        l = e;
    }
    (*group_seg)[LBM_MAX_GROUPS] = (int32_t)seg_begin->size();
    if (l != n) throw std::runtime_error("internal: links are not ordered by group");
    seg_begin->push_back(n);
}

Layout make_layout(const lbm_params* p, bool solids, int64_t n_links)
{
    Layout L{};
    const int64_t n = (int64_t)p->nx * p->ny * p->nz;
    int64_t ef = 0, eg = 0, g_in_f = -1;
    tile_geometry(p, &L.tiles, &ef, &eg, &g_in_f);
    const size_t es = (size_t)p->dtype;
    const size_t fb = align_up((size_t)ef * es);
    const size_t gb = p->thermal ? align_up((size_t)eg * es) : 0;
    const bool ab = p->streaming == LBM_STREAM_AB || p->streaming == LBM_STREAM_AB_PUSH;
    size_t off = 0;
    L.f = off; off += fb;
    L.g = off; off += gb;
    L.f2 = off; off += ab ? fb : 0;
    L.g2 = off; off += ab ? gb : 0;
    if (g_in_f >= 0) {
        // the temperature planes share the flow planes' tiles
        L.g = L.f + (size_t)g_in_f * es;
        L.g2 = L.f2 + (size_t)g_in_f * es;
    }
    L.mask = off; off += solids ? align_up(4 * (size_t)(mask_words(n) + (n + 31) / 32)) : 0;
    L.lcell = off; off += align_up(4 * (size_t)n_links);
    L.lcellw = off; off += align_up(4 * (size_t)n_links);
    L.lmeta = off; off += align_up(4 * (size_t)n_links);
    L.scratch = off; off += align_up(es * (size_t)n_links);
    int64_t face_off[6];
    L.face_vel = off; off += align_up(es * (size_t)face_planes(p, face_off));
    L.wall_T = off; off += align_up(8 * LBM_MAX_GROUPS);
    L.accum = off; off += align_up(8 * 4 * LBM_MAX_GROUPS);
    const size_t max_seg = max_segments(n_links);
    L.seg_begin = off; off += align_up(8 * (max_seg + 1));
    L.group_seg = off; off += align_up(4 * (LBM_MAX_GROUPS + 1));
    L.seg_sum = off; off += align_up(8 * 4 * max_seg);
    L.diag = off; off += align_up(8 * LBM_DIAG_COUNT);
    L.unstable = off; off += ALIGN;
    L.total = off;
    return L;
}

lbm_status device_error(lbm_ctx* ctx, hipError_t e, const char* what)
{
    ctx->err = std::string(what) + ": " + hipGetErrorString(e);
    return LBM_E_DEVICE;
}

#define LBM_HIP(ctx, call, what)                              \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return device_error(ctx, e_, what); \
    } while (0)

// ------------------------------------------------------- kernel timing

hipError_t take_event(lbm_ctx* c, hipEvent_t* ev)
{
    if (!c->spare_events.empty()) {
        *ev = c->spare_events.back();
        c->spare_events.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(ev);
}

// Record the start of a timed launch of `kind` on `stream`.
hipError_t timed_begin(lbm_ctx* c, hipStream_t stream, int kind)
{
    lbm_ctx::Timed t{kind, nullptr, nullptr};
    hipError_t e = take_event(c, &t.start);
    if (e != hipSuccess) return e;
    e = take_event(c, &t.stop);
    if (e != hipSuccess) {
        c->spare_events.push_back(t.start);
        return e;
    }
    c->timed.push_back(t);
    return hipEventRecord(t.start, stream);
}

hipError_t timed_end(lbm_ctx* c, hipStream_t stream) { return hipEventRecord(c->timed.back().stop, stream); }

// Add the recorded launches to the sums (synchronises the stream) and keep
// their events for reuse.
hipError_t add_up_timed(lbm_ctx* c)
{
    if (c->timed.empty()) return hipSuccess;
    hipError_t e = hipStreamSynchronize(c->stream);
    for (const lbm_ctx::Timed& t : c->timed) {
        if (e == hipSuccess) {
            float ms = 0.0f;
            e = hipEventElapsedTime(&ms, t.start, t.stop);
            c->prof_ms[t.kind] += ms;
            c->prof_launches[t.kind] += 1;
        }
        c->spare_events.push_back(t.start);
        c->spare_events.push_back(t.stop);
    }
    c->timed.clear();
    return e;
}

// A launch, timed when profiling and launched on the caller's stream (graph
// captures run on a private stream and are never timed).
#define LBM_TIMED(ctx, stream, kind, call, what)                                       \
    do {                                                                               \
        const bool timed_ = timing && (ctx)->profile && (stream) == (ctx)->stream;     \
        if (timed_) LBM_HIP(ctx, timed_begin(ctx, stream, kind), "profile event");     \
        LBM_HIP(ctx, call, what);                                                      \
        if (timed_) LBM_HIP(ctx, timed_end(ctx, stream), "profile event");             \
    } while (0)

// Where a step's kernels keep their per-call scratch: the gathered link
// values (link passes) and the force pass's per-segment sums.  Normally the
// context's own buffer; lbm_step_noalloc points them into the library's
// static device array.
struct StepScratch {
    char* links;
    double* seg_sum;
};

StepScratch own_scratch(const lbm_ctx* c) { return StepScratch{c->scratch, c->seg_sum}; }

template <typename R>
LinkArgs<R> link_args(lbm_ctx* c, int mode, char* fsrc, char* fdst, char* gsrc, char* gdst, const StepScratch& sc)
{
    LinkArgs<R> a{};
    a.geo = c->geo;
    a.cell = c->lcell;
    a.cellw = c->lcellw;
    a.meta = c->lmeta;
    a.scratch = (R*)sc.links;
    a.wall_T = c->wall_T;
    a.accum = c->accum;
    a.f_src = (R*)fsrc;
    a.f_dst = (R*)fdst;
    a.g_src = (R*)gsrc;
    a.g_dst = (R*)gdst;
    a.begin = 0;
    a.end = c->n_f + c->n_g;
    a.omega = abb_omega(&c->p);
    a.mode = mode;
    a.in_kernel = c->in_kernel ? 1 : 0;
    a.bb = make_bounce<R>(&c->p, c->in_kernel, c->face_vel);
    a.seg_begin = c->seg_begin;
    a.group_seg = c->group_seg;
    a.seg_sum = sc.seg_sum;
    a.n_seg = c->n_seg;
    return a;
}

template <typename R>
const Collision<R>& collision(const lbm_ctx* c);
template <>
const Collision<float>& collision<float>(const lbm_ctx* c) { return c->colf; }
template <>
const Collision<double>& collision<double>(const lbm_ctx* c) { return c->cold; }

// Enqueue one time step (parity from c->t) on `stream` and advance c->t;
// `last` adds the force/heat pass of a submission's last step.  `sc` names
// the step's scratch; `timing` = false never times the launches.
template <class L, typename R>
lbm_status enqueue_step(lbm_ctx* c, hipStream_t stream, bool last, const StepScratch& sc, bool timing = true)
{
    const int64_t n_links = c->n_f + c->n_g;
    const bool passes = !c->in_kernel && n_links > 0;
    const int parity = (int)(c->t & 1);
    StepArgs<R> s{};
    s.geo = c->geo;
    s.col = collision<R>(c);
    s.mask = c->mask;
    s.bb = make_bounce<R>(&c->p, c->in_kernel, c->face_vel);
    LinkArgs<R> la;
    if (!c->ab) {
        // one in-place kernel: collision, streaming (and bounce-back)
        s.f = (R*)c->f;
        s.g = (R*)c->g;
        s.parity = parity;
        LBM_TIMED(c, stream, parity ? LBM_KERNEL_STEP_ODD : LBM_KERNEL_STEP_EVEN,
                  (launch_aa_step<L, R>(s, c->thermal, c->lds[parity], stream)), "AA step kernel");
        la = link_args<R>(c, parity == 0 ? LINK_AA_AFTER_EVEN : LINK_AA_AFTER_ODD, c->f, c->f, c->g, c->g, sc);
        if (passes) {
            // link passes: gather every source, then scatter
            la.begin = 0;
            la.end = n_links;
            LBM_TIMED(c, stream, LBM_KERNEL_LINK_GATHER, launch_link_gather<R>(la, stream), "link gather kernel");
            LBM_TIMED(c, stream, LBM_KERNEL_LINK_SCATTER, launch_link_scatter<R>(la, stream), "link scatter kernel");
        }
    } else {
        char* fa = parity ? c->f2 : c->f;
        char* fb = parity ? c->f : c->f2;
        char* ga = parity ? c->g2 : c->g;
        char* gb = parity ? c->g : c->g2;
        s.f = (R*)fa;
        s.g = (R*)ga;
        s.f2 = (R*)fb;
        s.g2 = (R*)gb;
        if (c->push) {
            // one pass: collide, push and the boundary rules (links are always in the kernel)
            LBM_TIMED(c, stream, parity ? LBM_KERNEL_STEP_ODD : LBM_KERNEL_STEP_EVEN,
                      (launch_ab_push<L, R>(s, c->thermal, c->lds[parity], stream)), "A-B push kernel");
        } else {
            LBM_TIMED(c, stream, LBM_KERNEL_AB_COLLIDE, (launch_ab_collide<L, R>(s, c->thermal, c->lds[0], stream)),
                      "A-B collide kernel");
            LBM_TIMED(c, stream, LBM_KERNEL_AB_PULL, (launch_ab_pull<L, R>(s, c->thermal, c->lds[1], stream)),
                      "A-B pull kernel");
        }
        la = link_args<R>(c, LINK_AB, fa, fb, ga, gb, sc);
        if (passes) {
            // sources in one buffer, destinations in the other: one pass
            la.begin = 0;
            la.end = n_links;
            LBM_TIMED(c, stream, LBM_KERNEL_LINK_DIRECT, launch_link_direct<R>(la, stream), "link kernel");
        }
    }
    if (last) {
        // forces and heat of the submission's last step, read where each
        // link's bounced population was left
        const bool timed = timing && c->profile && stream == c->stream;
        if (timed) LBM_HIP(c, timed_begin(c, stream, LBM_KERNEL_FORCE), "profile event");
        la.begin = 0;
        la.end = n_links;
        LBM_HIP(c, (launch_link_force<L, R>(la, stream)), "force kernel");
        if (timed) LBM_HIP(c, timed_end(c, stream), "profile event");
    }
    c->t += 1;
    return LBM_OK;
}

// Capture 8 even/odd step pairs (kernel arguments and all) as one graph,
// once per context, at lbm_create.  Replays of 16 steps measured 0.4-1.7 %
// faster than of 2 steps on boxes of 4 M to 67 M cells (no slower on any),
// the gaps between graph launches being a larger share of a short step.  Any
// failure leaves the context on per-step launches.
template <class L, typename R>
void capture_pair(lbm_ctx* c)
{
    if (c->pair || c->pair_failed) return;
    c->pair_failed = true;
    if (hipStreamCreateWithFlags(&c->capture_stream, hipStreamNonBlocking) != hipSuccess) {
        c->capture_stream = nullptr;
        return;
    }
    const int64_t t_saved = c->t;
    const std::string err_saved = c->err;
    c->t = 0;
    hipGraph_t graph = nullptr;
    const int steps = 16;
    bool ok = hipStreamBeginCapture(c->capture_stream, hipStreamCaptureModeThreadLocal) == hipSuccess;
    if (ok) {
        bool launched = true;
        for (int i = 0; i < steps && launched; ++i)
            launched = enqueue_step<L, R>(c, c->capture_stream, false, own_scratch(c)) == LBM_OK;
        ok = hipStreamEndCapture(c->capture_stream, &graph) == hipSuccess && launched && graph;
    }
    c->t = t_saved;
    c->err = err_saved;
    hipGraphExec_t exec = nullptr;
    if (ok && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess) {
        // move the graph's work to the device now, not at its first launch
        if (hipGraphUpload(exec, c->capture_stream) == hipSuccess &&
            hipStreamSynchronize(c->capture_stream) == hipSuccess) {
            c->pair = exec;
            c->pair_steps = steps;
            c->pair_failed = false;
        } else {
            (void)hipGraphExecDestroy(exec);
        }
    }
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipGetLastError();  // a failed capture leaves no sticky error for the caller
}

// n steps: an odd first step alone, then replays of the step-pair graph,
// then the remaining steps (the very last with the force pass) launched
// directly.  Submissions of at most 17 steps launch every step directly.
template <class L, typename R>
lbm_status step_impl(lbm_ctx* c, int64_t n)
{
    int64_t left = n;
    if (c->profile) {
        // every kernel launched and timed on its own
        for (; left > 0; --left) {
            if (lbm_status st = enqueue_step<L, R>(c, c->stream, left == 1, own_scratch(c))) return st;
            if (c->timed.size() >= 1024) LBM_HIP(c, add_up_timed(c), "profile timing");
        }
        return LBM_OK;
    }
    if (c->pair && left > c->pair_steps + 1) {
        if (c->t & 1) {
            if (lbm_status st = enqueue_step<L, R>(c, c->stream, false, own_scratch(c))) return st;
            --left;
        }
        while (left > c->pair_steps) {
            LBM_HIP(c, hipGraphLaunch(c->pair, c->stream), "graph launch");
            c->t += c->pair_steps;
            left -= c->pair_steps;
        }
    }
    while (left > 0) {
        if (lbm_status st = enqueue_step<L, R>(c, c->stream, left == 1, own_scratch(c))) return st;
        --left;
    }
    return LBM_OK;
}

// n steps, each launched directly on the caller's stream with the step's
// scratch in `sc`; never timed, no graph.
template <class L, typename R>
lbm_status step_direct(lbm_ctx* c, int64_t n, const StepScratch& sc)
{
    for (int64_t left = n; left > 0; --left)
        if (lbm_status st = enqueue_step<L, R>(c, c->stream, left == 1, sc, false)) return st;
    return LBM_OK;
}

template <typename R>
FieldArgs<R> field_args(lbm_ctx* c)
{
    FieldArgs<R> a{};
    a.geo = c->geo;
    const bool second = c->ab && (c->t & 1);
    a.f = (R*)(second ? c->f2 : c->f);
    a.g = (R*)(second ? c->g2 : c->g);
    a.mask = c->mask;
    a.unstable = c->unstable;
    a.parity = (int32_t)(c->t & 1);
    a.ab = c->ab ? 1 : 0;
    a.bb = make_bounce<R>(&c->p, c->in_kernel, c->face_vel);
    a.col = collision<R>(c);
    return a;
}

// Scratch of lbm_step_noalloc: one static array per GPU, held until the
// process ends.  Host code never uses the name `scratch` as an address (on
// the host it names a stand-in): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept
// in noalloc_ptr.
static __device__ __align__(256) char scratch[LBM_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mutex;
void* noalloc_ptr[NOALLOC_MAX_DEVICES] = {};

// Device address of `scratch` on `dev` (looked up on the first call for that device).
hipError_t noalloc_scratch(int dev, void** out)
{
    *out = nullptr;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(noalloc_mutex);
    if (!noalloc_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        noalloc_ptr[dev] = ptr;
    }
    *out = noalloc_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t lbm_required_bytes(const lbm_params* p, const uint8_t* solid_labels)
{
    try {
        if (!validate(p).empty() || solid_on_slip_layer(p, solid_labels)) return 0;
        const bool solids = any_solid(p, solid_labels);
        const uint8_t* lab = solids ? solid_labels : nullptr;
        int64_t nl = build_links(p, lab, false, nullptr);
        if (p->thermal) nl += build_links(p, lab, true, nullptr);
        return make_layout(p, solids, nl).total;
    } catch (...) {
        return 0;
    }
}

lbm_status lbm_create(const lbm_params* p, const uint8_t* solid_labels, void* device_buf, size_t device_bytes,
                      void* hip_stream, lbm_ctx** out)
{
    if (out) *out = nullptr;
    g_create_error.clear();
    if (!out) {
        g_create_error = "out is NULL";
        return LBM_E_INVALID;
    }
    const std::string why = validate(p);
    if (!why.empty()) {
        g_create_error = why;
        return LBM_E_INVALID;
    }
    if (!device_buf) {
        g_create_error = "device_buf is NULL";
        return LBM_E_INVALID;
    }
    if (solid_on_slip_layer(p, solid_labels)) {
        g_create_error = "a solid cell lies in the first cell layer of a SLIP face";
        return LBM_E_INVALID;
    }
    lbm_ctx* c = nullptr;
    try {
        c = new lbm_ctx();
        c->p = *p;
        c->es = p->dtype;
        c->thermal = p->thermal != 0;
        c->ab = p->streaming == LBM_STREAM_AB || p->streaming == LBM_STREAM_AB_PUSH;
        c->push = p->streaming == LBM_STREAM_AB_PUSH;
        c->two_d = p->lattice == LBM_LATTICE_2D;
        c->stream = (hipStream_t)hip_stream;
        if (hipGetDevice(&c->device) != hipSuccess) c->device = 0;
        const bool solids = any_solid(p, solid_labels);
        const uint8_t* lab = solids ? solid_labels : nullptr;
        LinkList lf, lg;
        c->n_f = build_links(p, lab, false, &lf);
        c->n_g = c->thermal ? build_links(p, lab, true, &lg) : 0;
        const int64_t nl = c->n_f + c->n_g;
        const Layout L = make_layout(p, solids, nl);
        if (device_bytes < L.total) {
            g_create_error = "device_bytes " + std::to_string(device_bytes) + " < required " + std::to_string(L.total);
            delete c;
            return LBM_E_NOMEM;
        }
        if (((uintptr_t)device_buf) % ALIGN) {
            g_create_error = "device_buf must be 256-byte aligned";
            delete c;
            return LBM_E_INVALID;
        }
        Geometry& G = c->geo;
        G.nx = p->nx;
        G.ny = p->ny;
        G.nz = p->nz;
        G.nxy = p->nx * p->ny;
        G.ncell = G.nxy * p->nz;
        G.tile_lg = L.tiles.tile_lg;
        G.tile_mask = L.tiles.tile_mask;
        G.qstride = L.tiles.qstride;
        G.tile_f = L.tiles.tile_f;
        G.tile_g = L.tiles.tile_g;
        G.div_nx = make_magic((uint32_t)p->nx);
        G.div_ny = make_magic((uint32_t)p->ny);
        if (!magic_ok(G.div_nx, (uint32_t)G.ncell) || !magic_ok(G.div_ny, (uint32_t)G.ncell)) {
            g_create_error = "internal: division constants failed their self-check";
            delete c;
            return LBM_E_INVALID;
        }
        char* base = (char*)device_buf;
        c->f = base + L.f;
        c->g = c->thermal ? base + L.g : nullptr;
        c->f2 = c->ab ? base + L.f2 : nullptr;
        c->g2 = (c->ab && c->thermal) ? base + L.g2 : nullptr;
        c->mask = solids ? (uint32_t*)(base + L.mask) : nullptr;
        c->lcell = (int32_t*)(base + L.lcell);
        c->lcellw = (int32_t*)(base + L.lcellw);
        c->lmeta = (uint32_t*)(base + L.lmeta);
        c->scratch = base + L.scratch;
        c->face_vel = base + L.face_vel;
        c->wall_T = (double*)(base + L.wall_T);
        c->accum = (double*)(base + L.accum);
        c->seg_begin = (int64_t*)(base + L.seg_begin);
        c->group_seg = (int32_t*)(base + L.group_seg);
        c->seg_sum = (double*)(base + L.seg_sum);
        c->diag = (double*)(base + L.diag);
        c->unstable = (int32_t*)(base + L.unstable);
        c->colf = make_collision<float>(p);
        c->cold = make_collision<double>(p);
        const bool walls = nonperiodic(p, 0) || nonperiodic(p, 2) || nonperiodic(p, 4);
        c->in_kernel = p->links == LBM_LINKS_IN_KERNEL && (walls || solids);
        {
            int dev = 0, lds_cu = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
                lds_cu = 0;
            const int rules = boundary_rules(make_bounce<float>(p, c->in_kernel, nullptr));
            for (int k = 0; k < 2; ++k) {
                const int blocks =
                    p->occupancy[k] ? p->occupancy[k] : automatic_occupancy(p, c->ab, c->push, rules, k);
                c->lds[k] = occupancy_lds(blocks, lds_cu);
            }
        }

        // order the links of both lattices and upload
        LinkList all;
        c->n_wall = order_links(lf, lg, &all);
        lf = LinkList();
        lg = LinkList();
        std::vector<int32_t>& cell = all.cell;
        std::vector<int32_t>& cellw = all.cellw;
        std::vector<uint32_t>& meta = all.meta;
        std::vector<int64_t> seg_begin;
        std::vector<int32_t> group_seg;
        build_segments(meta, &seg_begin, &group_seg);
        c->n_seg = (int64_t)seg_begin.size() - 1;
        if ((size_t)c->n_seg > max_segments(nl)) throw std::runtime_error("internal: too many force segments");
        std::vector<double> wallT(LBM_MAX_GROUPS, 0.0);
        for (int f = 0; f < 6; ++f) wallT[f] = p->face_T[f];
        for (int gidx = 6; gidx < LBM_MAX_GROUPS; ++gidx) wallT[gidx] = p->solid_T;
        std::vector<uint32_t> mask;
        if (solids) mask = build_mask(p, solid_labels);
        {
            const std::string bad = check_link_destinations(p, all, solids ? &mask : nullptr, !c->in_kernel);
            if (!bad.empty()) {
                g_create_error = "internal: " + bad;
                delete c;
                return LBM_E_INVALID;
            }
        }
        // No byte of the buffer is left as the caller handed it over: every
        // population slot, padding and tile tails included, and the gathered
        // link values start as NaN (lbm_init_fields writes the slots the
        // cells own, so a read of a slot no cell owns shows in the fields);
        // the rest starts at zero, then takes the uploads.
        hipError_t e = launch_fill_words(base + L.f, L.mask - L.f, 0xffffffffu, c->stream);
        if (e == hipSuccess) e = launch_fill_words(base + L.mask, L.scratch - L.mask, 0u, c->stream);
        if (e == hipSuccess) e = launch_fill_words(base + L.scratch, L.face_vel - L.scratch, 0xffffffffu, c->stream);
        if (e == hipSuccess) e = launch_fill_words(base + L.face_vel, L.total - L.face_vel, 0u, c->stream);
        if (nl > 0) {
            if (e == hipSuccess) e = hipMemcpyAsync(c->lcell, cell.data(), 4 * nl, hipMemcpyHostToDevice, c->stream);
            if (e == hipSuccess) e = hipMemcpyAsync(c->lcellw, cellw.data(), 4 * nl, hipMemcpyHostToDevice, c->stream);
            if (e == hipSuccess) e = hipMemcpyAsync(c->lmeta, meta.data(), 4 * nl, hipMemcpyHostToDevice, c->stream);
        }
        std::vector<uint32_t> bits;
        if (solids) bits = near_bits(mask);
        if (e == hipSuccess && solids)
            e = hipMemcpyAsync(c->mask, mask.data(), 4 * (size_t)G.ncell, hipMemcpyHostToDevice, c->stream);
        if (e == hipSuccess && solids)
            e = hipMemcpyAsync(c->mask + mask_words(G.ncell), bits.data(), 4 * bits.size(), hipMemcpyHostToDevice,
                               c->stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(c->wall_T, wallT.data(), 8 * LBM_MAX_GROUPS, hipMemcpyHostToDevice, c->stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(c->seg_begin, seg_begin.data(), 8 * seg_begin.size(), hipMemcpyHostToDevice, c->stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(c->group_seg, group_seg.data(), 4 * group_seg.size(), hipMemcpyHostToDevice, c->stream);
        if (e == hipSuccess) e = launch_zero_f64(c->accum, 4 * LBM_MAX_GROUPS, c->stream);
        if (e == hipSuccess) e = launch_zero_f64((double*)c->unstable, 1, c->stream);  // flag sits in a 256-B slot
        // the host vectors die at return: wait for the copies
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
        if (e != hipSuccess) {
            g_create_error = std::string("upload: ") + hipGetErrorString(e);
            delete c;
            return LBM_E_DEVICE;
        }
        // the device address of lbm_step_noalloc's static scratch, looked up
        // here (once per device) so that no lbm_step_noalloc call does set-up
        // work, which a caller capturing it into a graph could not allow
        {
            void* noalloc_base = nullptr;
            e = noalloc_scratch(c->device, &noalloc_base);
            if (e != hipSuccess) {
                g_create_error = std::string("static scratch address: ") + hipGetErrorString(e);
                delete c;
                return LBM_E_DEVICE;
            }
        }
        // the replay graph of 16 steps, built once here (the pipeline creation
        // of "GPU lattice Boltzmann: streaming layout and performance", kept
        // out of the submissions that follow)
        if (c->two_d) c->es == 4 ? capture_pair<Lat2D, float>(c) : capture_pair<Lat2D, double>(c);
        else c->es == 4 ? capture_pair<Lat3D, float>(c) : capture_pair<Lat3D, double>(c);
        *out = c;
        return LBM_OK;
    } catch (const std::bad_alloc&) {
        g_create_error = "host allocation failed";
    } catch (const std::exception& ex) {
        g_create_error = ex.what();
    } catch (...) {
        g_create_error = "unknown error";
    }
    delete c;
    return LBM_E_INVALID;
}

lbm_status lbm_init_fields(lbm_ctx* c, const void* rho, const void* u, const void* T)
{
    if (!c) return LBM_E_INVALID;
    if (!rho || !u) {
        c->err = "rho and u are required";
        return LBM_E_INVALID;
    }
    c->t = 0;
    hipError_t e;
    if (c->es == 4) {
        FieldArgs<float> a = field_args<float>(c);
        a.rho = (const float*)rho;
        a.u = (const float*)u;
        a.T = (const float*)T;
        e = c->two_d ? launch_init<Lat2D, float>(a, c->thermal, c->stream)
                     : launch_init<Lat3D, float>(a, c->thermal, c->stream);
    } else {
        FieldArgs<double> a = field_args<double>(c);
        a.rho = (const double*)rho;
        a.u = (const double*)u;
        a.T = (const double*)T;
        e = c->two_d ? launch_init<Lat2D, double>(a, c->thermal, c->stream)
                     : launch_init<Lat3D, double>(a, c->thermal, c->stream);
    }
    if (e != hipSuccess) return device_error(c, e, "init kernel");
    // a fresh state: no forces of an earlier run, no unstable flag
    LBM_HIP(c, launch_zero_f64(c->accum, 4 * LBM_MAX_GROUPS, c->stream), "clear accumulators");
    LBM_HIP(c, launch_zero_f64((double*)c->unstable, 1, c->stream), "clear flag");
    c->initialised = true;
    return LBM_OK;
}

lbm_status lbm_step(lbm_ctx* c, int64_t n)
{
    if (!c) return LBM_E_INVALID;
    if (n < 0) {
        c->err = "n must be >= 0";
        return LBM_E_INVALID;
    }
    if (!c->initialised) {
        c->err = "lbm_init_fields has not been called";
        return LBM_E_INVALID;
    }
    if (n == 0) return LBM_OK;
    if (c->two_d) return c->es == 4 ? step_impl<Lat2D, float>(c, n) : step_impl<Lat2D, double>(c, n);
    return c->es == 4 ? step_impl<Lat3D, float>(c, n) : step_impl<Lat3D, double>(c, n);
}

lbm_status lbm_step_noalloc(lbm_ctx* c, int64_t n)
{
    if (!c) return LBM_E_INVALID;
    if (n < 0) {
        c->err = "n must be >= 0";
        return LBM_E_INVALID;
    }
    if (!c->initialised) {
        c->err = "lbm_init_fields has not been called";
        return LBM_E_INVALID;
    }
    // the step's scratch: gathered link values, then the force pass's segment sums
    const size_t links = (c->in_kernel || c->n_f + c->n_g == 0) ? 0 : align_up((size_t)c->es * (c->n_f + c->n_g));
    const size_t need = links + 8 * 4 * (size_t)c->n_seg;
    if (need > LBM_NOALLOC_SCRATCH_BYTES) {
        c->err = "lbm_step_noalloc: this context needs " + std::to_string(need) + " bytes of scratch, more than the " +
                 std::to_string((size_t)LBM_NOALLOC_SCRATCH_BYTES) + " the library holds per GPU (use lbm_step)";
        return LBM_E_INVALID;
    }
    if (n == 0) return LBM_OK;
    void* base = nullptr;
    LBM_HIP(c, noalloc_scratch(c->device, &base), "static scratch address");
    const StepScratch sc{(char*)base, (double*)((char*)base + links)};
    if (c->two_d) return c->es == 4 ? step_direct<Lat2D, float>(c, n, sc) : step_direct<Lat2D, double>(c, n, sc);
    return c->es == 4 ? step_direct<Lat3D, float>(c, n, sc) : step_direct<Lat3D, double>(c, n, sc);
}

lbm_status lbm_read_macros(lbm_ctx* c, void* rho, void* u, void* T)
{
    if (!c) return LBM_E_INVALID;
    if (!c->initialised) {
        c->err = "lbm_init_fields has not been called";
        return LBM_E_INVALID;
    }
    hipError_t e;
    if (c->es == 4) {
        FieldArgs<float> a = field_args<float>(c);
        a.rho_out = (float*)rho;
        a.u_out = (float*)u;
        a.T_out = (float*)T;
        e = c->two_d ? launch_read<Lat2D, float>(a, c->thermal, c->stream)
                     : launch_read<Lat3D, float>(a, c->thermal, c->stream);
    } else {
        FieldArgs<double> a = field_args<double>(c);
        a.rho_out = (double*)rho;
        a.u_out = (double*)u;
        a.T_out = (double*)T;
        e = c->two_d ? launch_read<Lat2D, double>(a, c->thermal, c->stream)
                     : launch_read<Lat3D, double>(a, c->thermal, c->stream);
    }
    if (e != hipSuccess) return device_error(c, e, "read kernel");
    return LBM_OK;
}

lbm_status lbm_wall_force(lbm_ctx* c, double* out, int32_t n_groups)
{
    if (!c) return LBM_E_INVALID;
    if (n_groups < 0 || (n_groups > 0 && !out)) {
        c->err = "bad output buffer";
        return LBM_E_INVALID;
    }
    std::vector<double> acc(4 * LBM_MAX_GROUPS, 0.0);
    int32_t unstable = 0;
    LBM_HIP(c, hipMemcpyAsync(acc.data(), c->accum, 8 * 4 * LBM_MAX_GROUPS, hipMemcpyDeviceToHost, c->stream),
            "copy accumulators");
    LBM_HIP(c, hipMemcpyAsync(&unstable, c->unstable, sizeof(int32_t), hipMemcpyDeviceToHost, c->stream),
            "copy flag");
    LBM_HIP(c, hipStreamSynchronize(c->stream), "synchronise");
    for (int32_t i = 0; i < n_groups; ++i)
        for (int k = 0; k < 4; ++k) out[4 * i + k] = i < LBM_MAX_GROUPS ? acc[4 * i + k] : 0.0;
    if (unstable) {
        c->err = "a fluid cell's rho, u or T was not finite at a read-back";
        return LBM_E_UNSTABLE;
    }
    return LBM_OK;
}

lbm_status lbm_diagnostics(lbm_ctx* c, double* out, int32_t n)
{
    if (!c) return LBM_E_INVALID;
    if (n < 0 || (n > 0 && !out)) {
        c->err = "bad output buffer";
        return LBM_E_INVALID;
    }
    if (!c->initialised) {
        c->err = "lbm_init_fields has not been called";
        return LBM_E_INVALID;
    }
    LBM_HIP(c, launch_zero_f64(c->diag, LBM_DIAG_COUNT, c->stream), "clear diagnostics");
    hipError_t e;
    if (c->two_d)
        e = c->es == 4 ? launch_diag<Lat2D, float>(field_args<float>(c), c->thermal, c->diag, c->stream)
                       : launch_diag<Lat2D, double>(field_args<double>(c), c->thermal, c->diag, c->stream);
    else
        e = c->es == 4 ? launch_diag<Lat3D, float>(field_args<float>(c), c->thermal, c->diag, c->stream)
                       : launch_diag<Lat3D, double>(field_args<double>(c), c->thermal, c->diag, c->stream);
    if (e != hipSuccess) return device_error(c, e, "diagnostics kernel");
    double d[LBM_DIAG_COUNT];
    int32_t unstable = 0;
    LBM_HIP(c, hipMemcpyAsync(d, c->diag, sizeof d, hipMemcpyDeviceToHost, c->stream), "copy diagnostics");
    LBM_HIP(c, hipMemcpyAsync(&unstable, c->unstable, sizeof(int32_t), hipMemcpyDeviceToHost, c->stream),
            "copy flag");
    LBM_HIP(c, hipStreamSynchronize(c->stream), "synchronise");
    d[LBM_DIAG_UMAX] = std::sqrt(d[LBM_DIAG_UMAX]);  // the kernel reduces |u|^2
    for (int32_t i = 0; i < n; ++i) out[i] = i < LBM_DIAG_COUNT ? d[i] : 0.0;
    if (unstable) {
        c->err = "a fluid cell's rho, u or T was not finite at a read-back";
        return LBM_E_UNSTABLE;
    }
    return LBM_OK;
}

int64_t lbm_time(const lbm_ctx* c) { return c ? c->t : -1; }

lbm_status lbm_resume(lbm_ctx* c, int64_t t)
{
    if (!c) return LBM_E_INVALID;
    if (t < 0) {
        c->err = "t must be >= 0";
        return LBM_E_INVALID;
    }
    // the buffer holds the state at time t in the layout of parity t & 1
    c->t = t;
    c->initialised = true;
    return LBM_OK;
}

int64_t lbm_count_links(const lbm_params* p, const uint8_t* solid_labels, int32_t lattice)
{
    try {
        if (!validate(p).empty() || solid_on_slip_layer(p, solid_labels)) return -1;
        const bool two_d = p->lattice == LBM_LATTICE_2D;
        const int flow = two_d ? 9 : 19, temp = two_d ? 5 : 7;
        if (lattice != flow && lattice != temp) return -1;
        const uint8_t* lab = any_solid(p, solid_labels) ? solid_labels : nullptr;
        return build_links(p, lab, lattice == temp, nullptr);
    } catch (...) {
        return -1;
    }
}

lbm_status lbm_check_links(const lbm_params* p, const uint8_t* solid_labels)
{
    g_create_error.clear();
    try {
        std::string why = validate(p);
        if (why.empty() && solid_on_slip_layer(p, solid_labels))
            why = "a solid cell lies in the first cell layer of a SLIP face";
        if (!why.empty()) {
            g_create_error = why;
            return LBM_E_INVALID;
        }
        const bool solids = any_solid(p, solid_labels);
        const uint8_t* lab = solids ? solid_labels : nullptr;
        LinkList lf, lg, all;
        build_links(p, lab, false, &lf);
        if (p->thermal) build_links(p, lab, true, &lg);
        order_links(lf, lg, &all);
        std::vector<uint32_t> mask;
        if (solids) mask = build_mask(p, solid_labels);
        const bool walls = nonperiodic(p, 0) || nonperiodic(p, 2) || nonperiodic(p, 4);
        const bool in_kernel = p->links == LBM_LINKS_IN_KERNEL && (walls || solids);
        const std::string bad = check_link_destinations(p, all, solids ? &mask : nullptr, !in_kernel);
        if (!bad.empty()) {
            g_create_error = "internal: " + bad;
            return LBM_E_INVALID;
        }
        return LBM_OK;
    } catch (const std::bad_alloc&) {
        g_create_error = "host allocation failed";
    } catch (const std::exception& ex) {
        g_create_error = ex.what();
    }
    return LBM_E_INVALID;
}

int64_t lbm_num_links(const lbm_ctx* c, int32_t lattice)
{
    if (!c) return -1;
    if (lattice == (c->two_d ? 9 : 19)) return c->n_f;
    if (lattice == (c->two_d ? 5 : 7)) return c->n_g;
    return -1;
}

lbm_status lbm_profile(lbm_ctx* c, int32_t on)
{
    if (!c) return LBM_E_INVALID;
    if (on != 0 && on != 1) {
        c->err = "on must be 0 or 1";
        return LBM_E_INVALID;
    }
    if (on) {
        // start the sums again; launches recorded before are dropped (their
        // events are re-recorded before they are read again)
        for (const lbm_ctx::Timed& t : c->timed) {
            c->spare_events.push_back(t.start);
            c->spare_events.push_back(t.stop);
        }
        c->timed.clear();
        for (int k = 0; k < LBM_KERNEL_KINDS; ++k) {
            c->prof_ms[k] = 0.0;
            c->prof_launches[k] = 0;
        }
    }
    c->profile = on != 0;
    return LBM_OK;
}

lbm_status lbm_profile_read(lbm_ctx* c, double* ms, int64_t* launches, int32_t n)
{
    if (!c) return LBM_E_INVALID;
    if (n < 0) {
        c->err = "n must be >= 0";
        return LBM_E_INVALID;
    }
    LBM_HIP(c, add_up_timed(c), "profile timing");
    for (int32_t k = 0; k < n; ++k) {
        if (ms) ms[k] = k < LBM_KERNEL_KINDS ? c->prof_ms[k] : 0.0;
        if (launches) launches[k] = k < LBM_KERNEL_KINDS ? c->prof_launches[k] : 0;
    }
    return LBM_OK;
}

const char* lbm_last_error(const lbm_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

void lbm_destroy(lbm_ctx* c)
{
    if (!c) return;
    // the queued steps may still read the caller's buffer and the graph
    (void)hipStreamSynchronize(c->stream);
    delete c;
}

}  // extern "C"
