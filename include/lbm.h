/*
 * lbm.h -- C ABI of the MI355X fused lattice Boltzmann time step.
 *
 * One library, liblbm_hip.so, built from hand-written HIP kernels for gfx950.
 * Every call takes plain pointers and sizes; no C++ or framework types cross
 * this boundary.  All compute runs in the library's kernels on the caller's
 * HIP stream; calls are stream-ordered and asynchronous except
 * lbm_wall_force(), lbm_diagnostics() and lbm_profile_read(), which
 * synchronise the stream (and lbm_step() while profiling, see lbm_profile()).
 *
 * What the library computes (the pages it follows):
 *  - "Multi-GPU thermal lattice Boltzmann simulations using OpenACC and MPI",
 *    Sec. 2: double-distribution thermal LB model, D3Q19 for the flow and D3Q7
 *    for the temperature, both with MRT collision; the force term
 *    F' = M^-1 (I - S/2) M F~ with F = rho g beta_T (T - T0) z;
 *    rho = sum f, u = (sum e f + F/2)/rho, T = sum g; half-way bounce-back
 *    f_ibar(x, t+dt) = f_i^+(x, t) for no-slip walls; half-way anti-bounce-back
 *    g_ibar(x, t+dt) = -g_i^+(x, t) + w T_w with w = (6 + a_T)/21 for a
 *    Dirichlet temperature wall and g_ibar = g_i^+ for an adiabatic one;
 *    Sec. 3: structure-of-arrays storage, population i of cell (x, y, z) at
 *    x + Nx*y + Nx*Ny*z + Nx*Ny*Nz*i.
 *  - "GPU lattice Boltzmann: streaming layout and performance" (OneCAD docs):
 *    one population buffer streamed in place with the AA pattern (even steps
 *    read (q, x) and write (opposite(q), x); odd steps read
 *    (opposite(q), x - c_q) and write (q, x + c_q)); coordinates computed once
 *    per cell and neighbours wrapped with a compare and an add; wall links
 *    handled by a gather pass into scratch followed by a scatter pass, with the
 *    momentum exchange taken in the gather of a submission's last step; the
 *    two-buffer layout (collide in place, then pull into the other buffer) as
 *    an option.
 *  - "GPU Optimization for High-Quality Kinetic Fluid Simulation", Sec. 3.1,
 *    Eq. 1-5: the lattice Boltzmann update as streaming plus collision with a
 *    force term, MRT relaxation Omega = -M^-1 D (m - m_eq).
 *
 * Readings of what the pages leave open (the library and its test oracle
 * follow the same readings, each in its own code):
 *  - D3Q19 = rest, 6 axis and 12 face-diagonal velocities; weights 1/3, 1/18,
 *    1/36; moment basis = the orthogonal basis of d'Humieres et al. with rows
 *    (in this order, which is the order of lbm_params.s19):
 *      0 rho: 1              1 e: 19c^2-30          2 eps: (21c^4-53c^2+24)/2
 *      3 jx: cx              4 qx: (5c^2-9)cx       5 jy, 6 qy, 7 jz, 8 qz
 *      9 3pxx: 3cx^2-c^2     10 3pixx: (3c^2-5)(3cx^2-c^2)
 *      11 pww: cy^2-cz^2     12 piww: (3c^2-5)(cy^2-cz^2)
 *      13 pxy: cx cy         14 pyz: cy cz          15 pxz: cx cz
 *      16 mx: (cy^2-cz^2)cx  17 my: (cz^2-cx^2)cy   18 mz: (cx^2-cy^2)cz
 *    m_eq = M f_eq with f_eq = w rho [1 + 3 c.u + 9/2 (c.u)^2 - 3/2 u.u];
 *    F~ = w [3 (c - u) + 9 (c.u) c] . F (Guo).
 *  - D3Q7 directions (0, +x, -x, +y, -y, +z, -z); rows of N (order of
 *    lbm_params.s7): 1, e_x, e_y, e_z, (-6,1,1,1,1,1,1), (0,2,2,-1,-1,-1,-1),
 *    (0,0,0,1,1,-1,-1); n_eq = (T, ux T, uy T, uz T, a_T T, 0, 0).
 *  - F = rho*accel + rho*gbeta*(T - T0) (gbeta a vector; buoyancy against
 *    gravity).  Initial state: f = f_eq(rho, u), g = N^-1 n_eq(T, u).
 *  - Momentum exchange on a wall link: the wall receives 2 c_p f_p^+; heat into
 *    the fluid through a Dirichlet link: w T_w - 2 g_p^+.
 *  - Walls sit half-way between the last fluid cell and the box face; a box
 *    face is periodic or one of the half-way kinds listed under the face
 *    kinds below, and an axis is periodic on both faces or on neither.  A
 *    link crossing two faces belongs to the first crossed axis in x, y, z
 *    order.
 */
#ifndef LBM_H
#define LBM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lbm_status {
    LBM_OK = 0,
    LBM_E_INVALID = 1,  /* bad argument; no device work was done */
    LBM_E_NOMEM = 2,    /* device_bytes smaller than lbm_required_bytes() */
    LBM_E_DEVICE = 3,   /* a HIP call failed; text in lbm_last_error() */
    LBM_E_UNSTABLE = 4, /* a fluid cell's rho or T was non-finite at a read-back */
} lbm_status;

/* Face kinds.  Every non-periodic face is a half-way boundary between the
 * last cell layer and the box face; a link (x, p) is a direction p of fluid
 * cell x that leaves through it.  "GPU lattice Boltzmann: streaming layout
 * and performance" names wall, reflection and open-face rules as per-link
 * rules without formulas; these are the textbook half-way forms (f values,
 * w_p the lattice weight, rho_w = face_rho, u_w = face_u of the face):
 *   WALL      f_opp(p)(x) = f_p^+(x)                       no-slip, at rest
 *             ("Multi-GPU thermal lattice Boltzmann ...", Sec. 2)
 *   SLIP      specular reflection: the normal part of c_p reverses and the
 *             tangential part c_t carries on, f_q(x + c_t) = f_p^+(x) with
 *             q = p reflected                              free slip
 *   VELOCITY  f_opp(p)(x) = f_p^+(x) - 6 w_p rho_w c_p.u_w  wall moving at
 *             u_w (Ladd): a velocity inlet, or a moving lid
 *   PRESSURE  f_opp(p)(x) = -f_p^+(x) + 2 w_p rho_w [1 + 9/2 (c_p.u)^2
 *             - 3/2 u.u], u the cell's own velocity in that step: an outlet
 *             held at density rho_w
 * A link leaving through two faces takes the rule of the first crossed axis
 * in x, y, z order, SLIP acting as WALL there.  The D3Q7 lattice takes each
 * non-periodic face's thermal rule (face_thermal) whatever its kind. */
enum { LBM_FACE_PERIODIC = 0, LBM_FACE_WALL = 1, LBM_FACE_SLIP = 2, LBM_FACE_VELOCITY = 3, LBM_FACE_PRESSURE = 4 };
enum { LBM_ADIABATIC = 0, LBM_DIRICHLET = 1 };
/* Streaming.  AA (AUTO): one population buffer, streamed in place with the
 * AA pattern.  AB: two buffers, the two passes of "GPU lattice Boltzmann:
 * streaming layout and performance" -- collide in place, then pull into the
 * other buffer (304 B per fp32 D3Q19 cell update).  AB_PUSH: two buffers in
 * one pass -- each cell loads its populations from one buffer, collides and
 * pushes them into the other (152 B per update, as AA); it applies the
 * boundary rules itself, so it needs links = LBM_LINKS_IN_KERNEL.  All three
 * give the same populations bit for bit. */
enum { LBM_STREAM_AUTO = 0, LBM_STREAM_AA = 1, LBM_STREAM_AB = 2, LBM_STREAM_AB_PUSH = 3 };
enum { LBM_MAX_GROUPS = 261 }; /* 6 faces + 255 solid labels */
/* Where half-way bounce-back happens.  IN_KERNEL: inside the step kernel (a
 * fluid cell next to a wall or solid re-reads and re-stores the bounced
 * populations in the odd step; solid cells are found from a per-cell mask,
 * walls from coordinates).  PASSES: the step kernel streams every cell as if
 * the box were periodic and separate link passes fix the blocked directions,
 * a gather of every link's source into scratch, then a scatter (the design of
 * "GPU lattice Boltzmann: streaming layout and performance").  Both give the
 * same populations bit for bit; IN_KERNEL moves fewer bytes. */
enum { LBM_LINKS_IN_KERNEL = 0, LBM_LINKS_PASSES = 1 };

/* Lattice pairs of the double-distribution model ("Multi-GPU thermal
 * lattice Boltzmann simulations using OpenACC and MPI", Sec. 2: D3Q19 + D3Q7
 * in three dimensions, D2Q9 + D2Q5 in two, MRT collision on both).
 *   LBM_LATTICE_3D  D3Q19 flow + D3Q7 temperature; rates s19, s7.
 *   LBM_LATTICE_2D  D2Q9 flow + D2Q5 temperature on a box with nz = 1 and
 *                   periodic z faces; rates s9, s5; accel[2], gbeta[2] and
 *                   the z components of face_u must be 0.  D2Q9 = rest, 4
 *                   axis and 4 diagonal velocities, weights 4/9, 1/9, 1/36;
 *                   moment basis of Lallemand and Luo, rows (order of s9):
 *                     0 rho: 1   1 e: 3c^2-4   2 eps: (9c^4-21c^2+8)/2
 *                     3 jx: cx   4 qx: (3c^2-5)cx   5 jy   6 qy
 *                     7 pxx: cx^2-cy^2   8 pxy: cx cy
 *                   D2Q5 directions (0, +x, -x, +y, -y), rows of N (order of
 *                   s5): 1, e_x, e_y, (-4,1,1,1,1), (0,1,1,-1,-1);
 *                   n_eq = (T, ux T, uy T, a_T T, 0); a_T in (-4, 1]; the
 *                   anti-bounce-back constant is w = (4 + a_T)/10 (Sec. 2).
 * Forces, heat and diagnostics keep their three components (z = 0 in 2D);
 * fields keep three velocity planes (uz = 0 in 2D; ignored by
 * lbm_init_fields). */
enum { LBM_LATTICE_3D = 0, LBM_LATTICE_2D = 1 };

/* Population layout in the device buffer (no effect on results, only on
 * speed).  Cells, in the order x + nx*(y + ny*z), are cut into tiles of 2^k
 * consecutive cells and each tile stores its planes one after another (the
 * collected structure of arrays of "GPU Optimization for High-Quality
 * Kinetic Fluid Simulation", Sec. 4.1); thermal boxes may keep the
 * temperature planes in the same tiles.  tile_log2 = 0 picks the layout
 * measured fastest on MI355X: tiles of 32 KiB per plane (2^13 fp32 or 2^12
 * fp64 cells; 64 KiB for isothermal fp32 D3Q19, 2^14 cells, and thermal fp64
 * D3Q19 + D3Q7, 2^13 cells) when the box holds at least four tiles, shared
 * tiles for thermal boxes except fp64 D2Q9 + D2Q5.  6..20 asks for
 * tiles of 2^k cells (shared for thermal boxes).  31 asks for one plane per
 * population over the whole box (the
 * structure of arrays of "Multi-GPU thermal lattice Boltzmann simulations
 * using OpenACC and MPI", Sec. 3).  Whatever is asked, a buffer that would
 * hold 2^32 elements or more tiled is stored one plane per population; the
 * automatic choice tiles a buffer of 4 GiB or more only where that measured
 * faster on MI355X (D3Q19 + D3Q7 in either precision, D2Q9 + D2Q5 in fp64). */

/* Occupancy of the step kernels (no effect on results, only on speed).
 * occupancy[0] governs the even steps (in place or AB_PUSH) and the collide
 * kernel of AB, occupancy[1] the odd steps and AB's pull kernel.  k in 1..8 lets at most k blocks of 256 cells run at once on one
 * compute unit (the launch reserves local data share that the kernel never
 * touches); -1 leaves the count to the kernel's register use; 0 picks the
 * value measured fastest on MI355X for the kernel instance (lattice,
 * precision, thermal or not, boundary rules compiled in) and -1 where none
 * was measured.  Fewer resident blocks keep fewer population streams open in
 * HBM at once, which favours the aligned, local accesses of the even step;
 * kernels whose loads wait on other loads (the boundary rules) need more
 * blocks to hide that latency. */

/* Faces are numbered 0..5 = x-, x+, y-, y+, z-, z+.  Force/heat group g is
 * face g for g < 6 and solid label g - 5 for g >= 6. */
typedef struct lbm_params {
    int32_t nx, ny, nz;      /* cells per axis, each >= 1; (nx*ny*nz + 1088) * dtype < 2^32 - 2^20 */
    int32_t dtype;           /* 4: fp32 populations and arithmetic, 8: fp64 */
    int32_t streaming;       /* LBM_STREAM_*; AUTO = in place (AA) */
    int32_t thermal;         /* 0: D3Q19 only, 1: D3Q19 + D3Q7 */
    int32_t face_kind[6];    /* LBM_FACE_*; an axis is periodic on both faces or on neither */
    int32_t face_thermal[6]; /* LBM_ADIABATIC or LBM_DIRICHLET (wall faces) */
    double face_T[6];        /* Dirichlet wall temperature per face */
    int32_t solid_thermal;   /* thermal rule of every solid cell */
    int32_t links;           /* LBM_LINKS_IN_KERNEL (0) or LBM_LINKS_PASSES (1), see above */
    double solid_T;          /* Dirichlet temperature of the solids */
    double s19[19];          /* D3Q19 relaxation rates, row order above, each in [0, 2) */
    double s7[7];            /* D3Q7 relaxation rates, row order above, each in [0, 2) */
    double a_T;              /* D3Q7 constant a_T (rest weight (1 - a_T)/7), in (-6, 1] */
    double accel[3];         /* body acceleration: F = rho*accel + ... */
    double gbeta[3];         /* buoyancy vector g*beta_T: F = ... + rho*gbeta*(T - T0) */
    double T0;               /* reference temperature of the buoyancy term */
    double face_u[6][3];     /* wall velocity u_w of each VELOCITY face */
    double face_rho[6];      /* wall density rho_w of each VELOCITY and PRESSURE face, > 0 */
    int32_t lattice;         /* LBM_LATTICE_3D (0) or LBM_LATTICE_2D (1), see above */
    int32_t pad1;
    double s9[9];            /* D2Q9 relaxation rates (LBM_LATTICE_2D), row order above, each in [0, 2) */
    double s5[5];            /* D2Q5 relaxation rates (LBM_LATTICE_2D), row order above, each in [0, 2) */
    int32_t tile_log2;       /* population layout, see above: 0 automatic, 6..20 tiles of 2^k cells, 31 none */
    int32_t pad2;
    int32_t occupancy[2];    /* resident blocks per compute unit, even / odd steps, see above: 0 automatic */
} lbm_params;

typedef struct lbm_ctx lbm_ctx;

/* Device bytes that lbm_create() needs for these parameters and labels:
 * population buffer(s), link arrays, link scratch, force accumulators and a
 * copy of the labels.  solid_labels: host, nx*ny*nz bytes in the order
 * x + nx*(y + ny*z), 0 = fluid, l >= 1 = solid of group 5 + l; NULL = no
 * solids.  Returns 0 if the parameters (or labels) are invalid. */
size_t lbm_required_bytes(const lbm_params* p, const uint8_t* solid_labels);

/* Validate the parameters, build the wall/solid link lists on the host
 * (every fluid cell x and direction p whose neighbour x + c_p is a wall face
 * or a solid cell), carve device_buf and upload the links.
 * Defined by: "Multi-GPU thermal lattice Boltzmann simulations using OpenACC
 * and MPI", Sec. 2 (the problem: a box of no-slip walls with half-way
 * bounce-back, Dirichlet walls with anti-bounce-back and adiabatic walls,
 * the relaxation matrices S and Q, the Boussinesq force) and "GPU lattice
 * Boltzmann: streaming layout and performance", streaming-layout section
 * (one population buffer in place or two buffers, per-link wall rules).
 * The links are checked before upload: no two links may store into one
 * slot and no solid cell's store may meet a fluid neighbour's bounce-back
 * store (see lbm_check_links); a failure is LBM_E_INVALID.
 * The step's replay graph (16 steps) is captured and instantiated here, once,
 * so that later submissions carry no set-up work (the page's "pipeline
 * creation", which it times apart from the steps).
 * device_buf: device memory of device_bytes bytes, 256-byte aligned,
 * BORROWED: the caller owns it and keeps it alive until lbm_destroy(); the
 * populations live in it, so saving its bytes and lbm_time() checkpoints the
 * state (lbm_resume).  Every population slot, padding included, is set to
 * NaN here; lbm_init_fields then writes the slots the cells own, so a read of
 * any other slot would show as NaN in the fields.
 * hip_stream: a hipStream_t (NULL = the null stream), BORROWED.
 * Host arrays are copied before the call returns.  On failure nothing is kept
 * and *out is NULL.  Errors: LBM_E_INVALID (bad sizes, a rate outside [0, 2),
 * a_T outside (-6, 1] (3D) or (-4, 1] (2D), one face of an axis periodic
 * and the other not, a 2D box with nz != 1 or non-periodic z faces or a
 * z component of accel, gbeta or face_u,
 * dtype not 4 or 8, a SLIP, VELOCITY or PRESSURE face with links =
 * LBM_LINKS_PASSES, a solid cell in the first layer of a SLIP face),
 * LBM_E_NOMEM (device_bytes too small), LBM_E_DEVICE. */
lbm_status lbm_create(const lbm_params* p, const uint8_t* solid_labels, void* device_buf,
                      size_t device_bytes, void* hip_stream, lbm_ctx** out);

/* Set the state to equilibrium of the given fields and the time to 0.
 * Defined by: "GPU Optimization for High-Quality Kinetic Fluid Simulation",
 * Sec. 3 (the initialisation step of its baseline GPU solver: populations,
 * density and velocity set up on the device before the first step; Eq. 2,
 * density and velocity as moments of f) and "Multi-GPU thermal lattice
 * Boltzmann simulations using OpenACC and MPI", Sec. 2 (the equilibrium
 * moments of both lattices).  The pages do not say which populations start
 * a run; the reading here is f = f_eq(rho, u), g = N^-1 n_eq(T, u).  The
 * latched forces and heat and the sticky unstable flag are cleared (a fresh
 * run).
 * rho: nx*ny*nz values, u: three planes (ux, uy, uz) of nx*ny*nz values,
 * T: nx*ny*nz values or NULL (thermal runs then start at T = 0); all device
 * pointers in the context's dtype, read by kernels enqueued on the stream.
 * Values on solid cells are ignored.  Asynchronous. */
lbm_status lbm_init_fields(lbm_ctx* ctx, const void* rho, const void* u, const void* T);

/* Enqueue n fused time steps (a "submission").  Defined by: "GPU lattice
 * Boltzmann: streaming layout and performance", streaming-layout section (the
 * AA pattern: even steps read (q, x) and write (opposite(q), x), odd steps
 * read (opposite(q), x - c_q) and write (q, x + c_q); submissions of many
 * steps; forces taken in the last step of a submission) and "Multi-GPU
 * thermal lattice Boltzmann simulations using OpenACC and MPI", Sec. 2
 * (the MRT collision of both lattices with the force term, half-way
 * bounce-back and anti-bounce-back).  Per step one in-place kernel
 * (collision + streaming of D3Q19 and, if thermal, D3Q7, with the half-way
 * bounce-back of wall and solid links inside it; with links =
 * LBM_LINKS_PASSES, link gather and scatter kernels after it instead).  The
 * forces and heat of the submission's last step are latched for
 * lbm_wall_force().
 * n = 0 is a no-op; n < 0 is LBM_E_INVALID.  Asynchronous. */
lbm_status lbm_step(lbm_ctx* ctx, int64_t n);

/* Bytes of the library's static per-GPU scratch used by lbm_step_noalloc. */
enum { LBM_NOALLOC_SCRATCH_BYTES = 16 << 20 };

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): lbm_step()
 * without allocation.  The same n steps with the same results bit for bit,
 * each kernel launched directly on the context's stream (no replay graph, no
 * per-kernel timing), and the step's per-call scratch -- the gathered link
 * values of LBM_LINKS_PASSES and the force pass's per-segment sums -- in a
 * static device array of LBM_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU until the process ends, instead of the context's buffer.
 * Calls no hipMalloc, hipFree or other allocating routine.  Every call on one
 * GPU shares that GPU's array and leaves its contents behind (each step
 * writes every scratch value it reads before reading it, so nothing needs
 * clearing); calls that overlap in time on one GPU (other streams, other
 * threads) race on it.  The array's device address is looked up by
 * lbm_create, so a call does no set-up work.  Under graph capture the graph
 * holds the launches of one call, with that call's step parities, while the
 * context's time (host state) advances once, at the call: capture an even
 * number of steps and set the time after replays with lbm_resume.  Errors:
 * LBM_E_INVALID (NULL context, n < 0, no lbm_init_fields, or a context whose
 * scratch exceeds the array: links * dtype for LBM_LINKS_PASSES plus 32
 * bytes per 1024 links of a group), LBM_E_DEVICE.  Asynchronous. */
lbm_status lbm_step_noalloc(lbm_ctx* ctx, int64_t n);

/* Macroscopic fields at the current time: rho, u = (sum c f + F/2)/rho as
 * three planes, T (may be NULL; ignored unless thermal).  Defined by:
 * "Multi-GPU thermal lattice Boltzmann simulations using OpenACC and MPI",
 * Sec. 2 (rho = sum f, u = (sum e f + F/2)/rho, T = sum g); the populations
 * are found where the AA pattern left them after an odd or an even step
 * count ("GPU lattice Boltzmann: streaming layout and performance").  Device pointers in
 * the context's dtype, written by a kernel on the stream.  Solid cells get
 * NaN.  If a fluid cell's rho or T is not finite, a sticky LBM_E_UNSTABLE is
 * recorded and returned by the next lbm_wall_force() or lbm_diagnostics().
 * Asynchronous. */
lbm_status lbm_read_macros(lbm_ctx* ctx, void* rho, void* u, void* T);

/* Copy the latched per-group sums of the last step of the last submission to
 * out (host, 4*n_groups doubles).  Defined by: "GPU lattice Boltzmann:
 * streaming layout and performance", streaming-layout section (momentum
 * exchange per wall link, taken at the step whose forces are read back) and
 * "Multi-GPU thermal lattice Boltzmann simulations using OpenACC and MPI",
 * Sec. 2 (the anti-bounce-back of a Dirichlet temperature link, through
 * which heat enters the fluid).  (Fx, Fy, Fz) = force on the face or solid,
 * the momentum the fluid hands over through its links, c_p f_out - c_in f_in
 * per link (2 c_p f_p^+ for a wall), Q = heat into the fluid through its
 * Dirichlet links.  Groups beyond
 * LBM_MAX_GROUPS are zero-filled.  The sums are taken in a fixed order (no
 * atomics), so the same state gives the same values bit for bit.
 * Synchronises the stream; returns LBM_E_UNSTABLE if a read-back saw a
 * non-finite fluid value. */
lbm_status lbm_wall_force(lbm_ctx* ctx, double* out, int32_t n_groups);

/* Indices of the values lbm_diagnostics() returns. */
enum {
    LBM_DIAG_FLUID_CELLS = 0, /* number of fluid cells */
    LBM_DIAG_MASS = 1,        /* sum of rho */
    LBM_DIAG_MOM_X = 2,       /* sum of rho u_x (u with the half force, as read back) */
    LBM_DIAG_MOM_Y = 3,
    LBM_DIAG_MOM_Z = 4,
    LBM_DIAG_KINETIC = 5,     /* sum of rho |u|^2 / 2 */
    LBM_DIAG_UMAX = 6,        /* max |u| */
    LBM_DIAG_HEAT = 7,        /* sum of T (0 unless thermal) */
    LBM_DIAG_CONV_X = 8,      /* sum of u_x T: advective heat flux (0 unless thermal) */
    LBM_DIAG_CONV_Y = 9,
    LBM_DIAG_CONV_Z = 10,
    LBM_DIAG_COUNT = 11
};

/* Volume diagnostics at the current time: sums over the fluid cells of the
 * fields lbm_read_macros() returns, accumulated in fp64 on the device, written
 * to out (host, n doubles; values past LBM_DIAG_COUNT are zero-filled).  They
 * give the heat-transfer figures of a convection cell heated through the two
 * faces of axis a, H cells apart (walls half-way, so H = the box extent),
 * with temperature difference dT and thermal diffusivity alpha:
 *   wall Nusselt number   Nu_w = Q * H / (alpha * dT * A), with Q the heat
 *                          through one heated face per step (lbm_wall_force)
 *                          and A its area in cells;
 *   volume Nusselt number Nu_v = 1 + <u_a T> * H / (alpha * dT), with
 *                          <u_a T> = out[LBM_DIAG_CONV_a] / fluid cells
 *                          (a box without solid cells).
 * At a steady state the hot and cold faces pass the same heat (Q_hot = -Q_cold),
 * and Nu_v agrees with Nu_w up to the discretisation.
 * Synchronises the stream; returns LBM_E_UNSTABLE if a fluid value was not
 * finite (then the sums are not finite either). */
lbm_status lbm_diagnostics(lbm_ctx* ctx, double* out, int32_t n);

/* Kernel kinds of per-kernel timing (lbm_profile_read). */
enum {
    LBM_KERNEL_STEP_EVEN = 0,    /* the step kernel at even t: in place (AA) or one-pass two buffers (AB_PUSH) */
    LBM_KERNEL_STEP_ODD = 1,     /* the same at odd t */
    LBM_KERNEL_AB_COLLIDE = 2,   /* two buffers in two passes (AB): collide in place */
    LBM_KERNEL_AB_PULL = 3,      /* ... then pull into the other buffer */
    LBM_KERNEL_LINK_GATHER = 4,  /* link passes (LBM_LINKS_PASSES), in place: gather */
    LBM_KERNEL_LINK_SCATTER = 5, /* ... then scatter */
    LBM_KERNEL_LINK_DIRECT = 6,  /* link passes with two buffers: one pass */
    LBM_KERNEL_FORCE = 7,        /* a submission's last step: clearing the sums and the force / heat pass */
    LBM_KERNEL_KINDS = 8
};

/* Per-kernel timing, the profile mode of "GPU lattice Boltzmann: streaming
 * layout and performance", which times each kernel with GPU timestamps and
 * warns that throughput is then not representative.  on = 1: the sums start
 * again at zero and, from the next lbm_step on, every kernel of a step is
 * launched on its own (no graph replays) between two HIP events recorded on
 * the stream; every 1024 timed launches lbm_step synchronises the stream to
 * add them up.  on = 0: back to normal launches; the sums stay readable.
 * Fields, forces and heat are the same bit for bit either way.  No device
 * work.  Errors: LBM_E_INVALID for a NULL context or on not 0 or 1. */
lbm_status lbm_profile(lbm_ctx* ctx, int32_t on);

/* Milliseconds and launch counts per kernel kind (LBM_KERNEL_*) timed since
 * profiling was last switched on: ms[k] and launches[k] for k < n (host
 * arrays, either may be NULL; kinds from LBM_KERNEL_KINDS on read 0).
 * Synchronises the stream.  Errors: LBM_E_INVALID (NULL context, n < 0),
 * LBM_E_DEVICE. */
lbm_status lbm_profile_read(lbm_ctx* ctx, double* ms, int64_t* launches, int32_t n);

/* Current time step count (number of steps since lbm_init_fields). */
int64_t lbm_time(const lbm_ctx* ctx);

/* Continue from a checkpoint.  A checkpoint is the device_bytes bytes of a
 * context's buffer, copied after its stream has finished a call, with that
 * context's lbm_time() t.  To resume: create a context with the same
 * parameters, labels, dtype and streaming mode, copy the saved bytes into its
 * buffer (on or ordered before its stream), then call lbm_resume(ctx, t) in
 * place of lbm_init_fields; the next lbm_step continues at step t exactly as
 * the saved context would have.  No device work.  Errors: LBM_E_INVALID for a
 * NULL context or t < 0. */
lbm_status lbm_resume(lbm_ctx* ctx, int64_t t);

/* Host only (no device work): build the links lbm_create() would build for
 * these parameters and labels and check them, as lbm_create() does: no two
 * links store into one slot (the returning populations of the bounce-back
 * inside the step kernel, and with links = LBM_LINKS_PASSES the stores of
 * the link passes after an even and after an odd step), and every solid cell
 * leaves the slot a fluid neighbour bounces into to that neighbour (its mask
 * bit).  The in-place step ("GPU lattice Boltzmann: streaming layout and
 * performance": each cell writes exactly the slots it read) relies on both.
 * Returns LBM_OK, or LBM_E_INVALID with the reason in lbm_last_error(NULL). */
lbm_status lbm_check_links(const lbm_params* p, const uint8_t* solid_labels);

/* Number of links of the flow lattice's list (lattice = 19 for D3Q19 or 9
 * for D2Q9) or of the temperature lattice's (7 for D3Q7, 5 for D2Q5); -1
 * when the number does not name a lattice of this context. */
int64_t lbm_num_links(const lbm_ctx* ctx, int32_t lattice);

/* Host only (no device work): the number of links lbm_create() would build
 * for these parameters and labels on the flow lattice (19 or 9) or the
 * temperature lattice (7 or 5) of p->lattice; a link is a fluid cell x and
 * direction p with x + c_p a wall face or a solid cell.  Returns -1 for
 * invalid parameters or lattice. */
int64_t lbm_count_links(const lbm_params* p, const uint8_t* solid_labels, int32_t lattice);

/* Last error text of this context (or of the last failed lbm_create when ctx
 * is NULL).  Valid until the next call on the same context. */
const char* lbm_last_error(const lbm_ctx* ctx);

/* Wait for the work queued on the context's stream, then release the
 * context (its host memory and its replay graph; device_buf stays the
 * caller's, who may free it once this returns).  NULL is ignored. */
void lbm_destroy(lbm_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* LBM_H */
