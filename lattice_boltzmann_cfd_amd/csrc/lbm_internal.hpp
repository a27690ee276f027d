// lbm_internal.hpp -- launch descriptors shared by the C-ABI host code and
// the kernels of liblbm_hip.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lbm.h"
#include "lbm_lattice.hpp"

namespace lbm {

// Unsigned division by a run-time constant d >= 1 for numerators < 2^31:
// n / d == (n * mul) >> shift with mul = ceil(2^(31+l) / d), shift = 31 + l,
// l = ceil(log2 d) (Granlund-Montgomery round-up method).
struct DivMagic {
    uint64_t mul;
    uint32_t shift;
    uint32_t d;
};

__host__ __device__ inline uint32_t divide(uint32_t n, const DivMagic& m)
{
    return (uint32_t)(((uint64_t)n * m.mul) >> m.shift);
}

// Box geometry as the kernels see it.
struct Geometry {
    int32_t nx, ny, nz;
    int32_t nxy;
    int32_t ncell;
    int32_t pad0;
    // population buffers: cells in tiles of 2^tile_lg consecutive cells, each
    // tile holding its planes one after another (tile_lg = 31: one tile, the
    // plain structure of arrays)
    int64_t qstride;     // elements between planes inside a tile
    uint32_t tile_f;     // elements between consecutive tiles of a flow-lattice buffer (< 2^24)
    uint32_t tile_g;     // elements between consecutive tiles of a temperature-lattice buffer (< 2^24)
    uint32_t tile_lg;
    uint32_t tile_mask;  // 2^tile_lg - 1
    DivMagic div_nx, div_ny;
};

// Link record (structure of arrays):
//   cell  : the fluid cell x of the link
//   cellw : the periodic image of x + c_p (where the population lands); for
//           a SLIP link the image of x + c_t (where the reflected population
//           lands, c_t the tangential part of c_p); for a PRESSURE link the
//           cell's index on its face (see Bounce::face_vel)
//   meta  : bits 0..4 direction p (kernel order of its lattice),
//           bits 5..13 force/heat group, bit 14 Dirichlet (D3Q7 only),
//           bit 15 the link belongs to the temperature lattice (D3Q7 or D2Q5),
//           bits 16..17 the D3Q19 rule (LinkRule), bits 18..19 the axis of
//           the governing face
// Links [0, n_wall) cross a box face; [n_wall, n_total) end in a solid cell.
// Each part is sorted by (group, lattice, direction, cell).
constexpr uint32_t LINK_DIR_MASK = 31u;
constexpr uint32_t LINK_GROUP_SHIFT = 5;
constexpr uint32_t LINK_GROUP_MASK = 511u;
constexpr uint32_t LINK_DIRICHLET = 1u << 14;
constexpr uint32_t LINK_TEMP = 1u << 15;
constexpr uint32_t LINK_RULE_SHIFT = 16;
constexpr uint32_t LINK_AXIS_SHIFT = 18;
enum LinkRule : uint32_t { RULE_WALL = 0, RULE_SLIP = 1, RULE_VELOCITY = 2, RULE_PRESSURE = 3 };

// Per-cell solid mask (only when the box has solid cells).  On a fluid cell,
// bit q (1..18, or 1..8 for D2Q9) is set when x + c_q is a solid cell reached
// without crossing a wall face (a solid link).  On a solid cell, MASK_SOLID is set and bit q
// marks that (s + c_q, opp q) is such a solid link of a fluid neighbour,
// which re-reads and re-stores the slot the solid cell's odd step would store
// direction q to.  Temperature direction k (D3Q7: 1..6, D2Q5: 1..4) is the
// flow lattice's axis direction k, so those bits serve both lattices.
// The mask words are followed (Bounce::near_off words after the first) by a
// bitmap of one bit per cell, set where the cell's mask word is not 0: the
// step kernels read that bit first (a wavefront's 64 bits are 8 bytes) and
// the 4-byte word only where it is set.
constexpr uint32_t MASK_SOLID = 1u << 31;

// Which slots a link pass reads and writes.
enum LinkMode : int32_t {
    LINK_AA_AFTER_EVEN = 0,  // src (opp p, x), dst (p, x + c_p)
    LINK_AA_AFTER_ODD = 1,   // src (p, x + c_p), dst (opp p, x)
    LINK_AB = 2,             // src A(p, x) post-collision, dst B(opp p, x)
};

// Boundary constants of the in-kernel boundary handling.  Faces are numbered
// 0..5 = x-, x+, y-, y+, z-, z+; walls[f] is set for every non-periodic face,
// and slip / vel / pres mark the faces of those kinds (the rest of the
// non-periodic faces are no-slip walls).  A D3Q7 population bouncing off face
// f becomes gw[f] - g (anti-bounce-back, Dirichlet face) or g (adiabatic);
// off a solid, solid_gw - g or g.
template <typename R>
struct Bounce {
    R face_gw[6];
    R solid_gw;
    int32_t walls;            // bit f: face f is not periodic
    int32_t face_dirichlet;   // bit f: face f has a Dirichlet temperature
    int32_t solid_dirichlet;  // solids have a Dirichlet temperature
    int32_t in_kernel;        // walls and solids are handled inside the step kernel
    int32_t slip, vel, pres;  // bit f: face f is a SLIP / VELOCITY / PRESSURE face
    int32_t near_off;         // boxes with solids: words from the mask to its bitmap of cells with mask != 0
    R face_rho[6];            // wall density (VELOCITY, PRESSURE faces)
    R face_u[6][3];           // wall velocity (VELOCITY faces)
    // PRESSURE faces: the velocity of every cell of the face in its last
    // step, three planes (ux, uy, uz) of face_area[f] values starting at
    // face_vel + face_off[f]; a cell's index on an x face is y + ny z, on a y
    // face x + nx z, on a z face x + nx y.
    R* face_vel;
    int64_t face_off[6];
    int64_t face_area[6];
};

template <typename R>
struct StepArgs {
    Geometry geo;
    R* f;  // D3Q19 populations (AA: the only buffer; AB: source/in-place buffer)
    R* g;  // D3Q7 populations or null
    R* f2; // AB: destination buffer of the pull
    R* g2;
    const uint32_t* mask;  // solid mask, or null when the box has no solid cell
    Bounce<R> bb;
    int32_t parity;
    int32_t pad0;
    Collision<R> col;
};

template <typename R>
struct LinkArgs {
    Geometry geo;
    const int32_t* cell;
    const int32_t* cellw;
    const uint32_t* meta;
    R* scratch;
    const double* wall_T;  // per group: Dirichlet temperature
    double* accum;         // per group: Fx, Fy, Fz, Q
    R* f_src;
    R* f_dst;
    R* g_src;
    R* g_dst;
    int64_t begin;  // first link of the launch
    int64_t end;    // one past the last link of the launch
    double omega;          // (6 + a_T)/21
    int32_t mode;
    int32_t in_kernel;     // bounce-back happened inside the step kernel
    Bounce<R> bb;          // face rules and the PRESSURE faces' velocities
    // force pass: the links cut into segments of one group each, at most
    // LINK_SEGMENT links long; segment k is links [seg_begin[k], seg_begin[k + 1])
    // and group g owns segments [group_seg[g], group_seg[g + 1])
    const int64_t* seg_begin;
    const int32_t* group_seg;
    double* seg_sum;  // per segment: Fx, Fy, Fz, Q
    int64_t n_seg;
};

// Links per force-pass segment: one wavefront sums a segment, 16 links a lane.
constexpr int64_t LINK_SEGMENT = 1024;

template <typename R>
struct FieldArgs {
    Geometry geo;
    R* f;
    R* g;
    const uint32_t* mask;  // solid mask, or null when there are no solids
    const R* rho;
    const R* u;
    const R* T;
    R* rho_out;
    R* u_out;
    R* T_out;
    int32_t* unstable;
    int32_t parity;
    int32_t ab;  // populations in natural layout (two-buffer mode)
    Bounce<R> bb;
    Collision<R> col;
};

// Boundary rules compiled into a cell kernel instance: 0 none (periodic box,
// or bounce-back left to the link passes), 1 walls and solids, 2 also SLIP,
// VELOCITY or PRESSURE faces.
template <typename R>
inline int boundary_rules(const Bounce<R>& b)
{
    return b.in_kernel ? ((b.slip | b.vel | b.pres) ? 2 : 1) : 0;
}

// Launch wrappers (defined in lbm_kernels.hip).  Each returns the HIP error
// of the launch.  L is the lattice pair (Lat3D: D3Q19 + D3Q7, Lat2D: D2Q9 +
// D2Q5 on one z layer); the link gather / scatter passes do not depend on it.
// `lds`: bytes of local data share reserved per block and never used, which
// bounds the blocks resident on one compute unit (0: no reservation).
template <class L, typename R>
hipError_t launch_aa_step(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s);
template <class L, typename R>
hipError_t launch_ab_collide(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s);
template <class L, typename R>
hipError_t launch_ab_pull(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s);
template <class L, typename R>
hipError_t launch_ab_push(const StepArgs<R>& a, bool thermal, size_t lds, hipStream_t s);
template <typename R> hipError_t launch_link_gather(const LinkArgs<R>& a, hipStream_t s);
template <typename R> hipError_t launch_link_scatter(const LinkArgs<R>& a, hipStream_t s);
template <typename R> hipError_t launch_link_direct(const LinkArgs<R>& a, hipStream_t s);
template <class L, typename R> hipError_t launch_link_force(const LinkArgs<R>& a, hipStream_t s);
template <class L, typename R> hipError_t launch_init(const FieldArgs<R>& a, bool thermal, hipStream_t s);
template <class L, typename R> hipError_t launch_read(const FieldArgs<R>& a, bool thermal, hipStream_t s);
// Volume sums of lbm_diagnostics() into out[LBM_DIAG_COUNT] (cleared by the caller).
template <class L, typename R>
hipError_t launch_diag(const FieldArgs<R>& a, bool thermal, double* out, hipStream_t s);
hipError_t launch_zero_f64(double* p, int64_t n, hipStream_t s);
// Every 32-bit word of [p, p + bytes) set to `word` (0xffffffff: a NaN in
// fp32 and fp64); p and bytes multiples of 16.
hipError_t launch_fill_words(void* p, size_t bytes, uint32_t word, hipStream_t s);

}  // namespace lbm
