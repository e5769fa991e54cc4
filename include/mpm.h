/*
 * mpm.h -- C ABI of libmpm, the MI355X (gfx950) particle-to-grid (P2G) hot
 * path of the material point method and the steps around it.
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; the caller owns them (the library allocates nothing
 *    and keeps no per-call state between calls; the one exception is the
 *    static scratch of mpm_p2g_isplit_noalloc).  Host pointers are read
 *    before the call returns.
 *  - Work is enqueued on `stream` and the call returns without waiting; the
 *    library never synchronises the stream.  Results (and the status
 *    counters) are valid once the caller's stream has reached that point.
 *  - The return value reports only errors the host can detect before any
 *    launch (bad descriptor, NULL or misaligned pointer, workspace too small,
 *    bounds that would overflow) or a failed launch.  On a non-zero return
 *    nothing was enqueued, except for MPM_ERR_HIP after a partial launch
 *    sequence, which leaves outputs unspecified.
 *  - Conditions met on the device are counted in the caller's status
 *    counters (uint32_t status[4], zeroed by the caller, accumulated into):
 *      status[0]  particles skipped because their stencil leaves the grid
 *                 (or a coordinate is not finite),
 *      status[1]  particles skipped because mass, velocity or affine entries
 *                 fall outside the declared ranges the bounds check proved,
 *      status[2]  particles whose advected position was clamped to the box,
 *      status[3]  internal consistency faults: an order entry naming no
 *                 particle, or a binned record outside its tile (skipped;
 *                 0 in correct use).
 *    "Implementation -- GPU Optimization & Reference Codebases", section 5
 *    rules 8 and 9: read back asynchronously, and count what overflows or is
 *    clamped instead of sanitising silently.
 *  - Layouts are component-major structure-of-arrays: a per-particle vector
 *    field of D components over N particles is float[D][N]; the affine
 *    matrix is float[dim*dim][N] with entry (row d, column e) at
 *    [(d*dim + e)*N + p].  Grids are int64[channels][n]...[n] with x fastest;
 *    channel 0 is mass, channel 1+d momentum along axis d.
 */
#ifndef MPM_H
#define MPM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MPM_OK = 0,
    MPM_ERR_INVALID = -1,   /* bad descriptor, NULL or misaligned pointer, bad size */
    MPM_ERR_OVERFLOW = -2,  /* the declared ranges could overflow the accumulators */
    MPM_ERR_DOMAIN = -3,    /* reserved: domain problems are counted on the device */
    MPM_ERR_WORKSPACE = -4, /* workspace smaller than mpm_workspace_bytes() */
    MPM_ERR_HIP = -6,       /* a HIP call or kernel launch failed */
    MPM_ERR_SCRATCH = -7    /* the input needs more than the library's static scratch holds */
} mpm_status;

/* The background grid of the quadratic-stencil transfer.  The domain is the
 * unit square/cube with n nodes per axis, node i at i/n (dx = 1/n).
 * n must be a power of two in [8, 1024] (2D) or [8, 512] (3D), so that x*n
 * and dx are exact in float32.  Fixed-point scale S = 2^frac_bits with
 * frac_bits in [0, 60].  tile is the binning tile edge in cells and must be 4. */
typedef struct {
    int32_t dim;
    int32_t n;
    int32_t frac_bits;
    int32_t tile;
} mpm_grid_desc;

/* Particle attributes, device pointers, component-major (see above).
 * C may be NULL for a transfer without the affine term (treated as zero). */
typedef struct {
    int64_t n;
    float *x;     /* [dim][n] positions in the unit domain */
    float *v;     /* [dim][n] velocities */
    float *C;     /* [dim*dim][n] affine (APIC) matrices */
    float *m;     /* [n] masses */
} mpm_particles;

/* Declared ranges: |m| <= max_mass, |v_d| <= max_speed, |C_de| <= max_affine.
 * The bounds check proves that no accumulator can overflow for particles in
 * these ranges; a particle outside them is skipped and counted (status[1]).
 * "particle to grid transfer in checked integer arithmetic", section "the
 * program": the bounds line runs before any particle is scattered. */
typedef struct {
    double max_mass;
    double max_speed;
    double max_affine;
} mpm_ranges;

/* Offsets (bytes from the workspace base) of the arrays mpm_bin_particles
 * writes, so that callers and tests can read them.  Counts are the
 * capacities allocated, not what one call fills. */
typedef struct {
    size_t tile_count;      /* uint32 [n_tiles]     binned particles per tile                    */
    size_t tile_start;      /* uint32 [n_tiles + 1] first record of each tile (exclusive prefix sum) */
    size_t tile_active;     /* uint8  [n_tiles] written by mpm_grid_update and mpm_grid_clear when
                                        given the bins: 1 for the node tiles that P2G from these
                                        bins can reach */
    size_t meta;            /* uint32 [32]: [0] items, [2] binned particles, [3] work cursor,
                                        [6] runs (chunk, tile) of the count, [7] cell keys written,
                                        [16..24] the binning's stamp
                                        (grid, particle count, declared ranges, resident or
                                        checked), which every reader of the bins compares with
                                        its own arguments on the device.  (Offsets up to here do
                                        not depend on the particle count.) */
    size_t items;           /* uint32 [max_items][4] work items: tile, first record, records (a
                                        slice of at most rows_per_item rows' worth of a tile's
                                        records), 0; handed out alternately the largest and
                                        smallest remaining                                 */
    size_t rank;            /* uint32 [n] rank of each particle inside its tile (internal)      */
    size_t slot;            /* uint32 [n] record index of each particle (0xFFFFFFFF: not binned) */
    size_t cell_key;        /* uint8  [n + 4] local cell number of each record, in record order, written
                                        when meta[7] is 1 (the binning's runs averaged at least 32
                                        records); otherwise mpm_p2g reads a record's cell from its
                                        position */
    size_t sorted;          /* float  [n][n_fields] binned records x, v, C, m (+ padding floats),
                                        tile by tile                                       */
    size_t scan_tmp;        /* uint32 [ceil(n_tiles/4096)][2 + rows_per_item] per-block sums of the
                                        work-item plan (internal)                          */
    int64_t n_cells, n_tiles, max_items, n_fields, rows_per_item;
    size_t total_bytes;
} mpm_ws_layout;

/* ------------------------------------------------------------------------ */

/* Library version string (static storage). */
const char *mpm_version(void);

/* Message for a return code (static storage). */
const char *mpm_strerror(int code);

/* Host-only bounds line, run before any scatter ("particle to grid transfer
 * in checked integer arithmetic", sections "integers do not care about
 * order" and "limits").  The largest quantised contribution is
 *   S * (3/4)^dim * max_mass * max(1, max_speed + dim * max_affine * 1.5 dx)
 * (each 1D quadratic weight is at most 3/4, each node offset at most 1.5
 * cells), plus float32 rounding.  Returns MPM_OK when n_particles times that
 * stays below 2^63 (every int64 node sum completes in any order) and one
 * P2G work item's worth of it stays below 2^53 (the exact float64 on-chip
 * partial sums), else MPM_ERR_OVERFLOW.  log2_bound (may be NULL) receives
 * log2(n_particles * largest contribution). */
int mpm_check_bounds(const mpm_grid_desc *grid, int64_t n_particles, const mpm_ranges *ranges,
                     double *log2_bound);

/* Workspace size for binning n_particles on this grid (host-only): the
 * histogram, prefix sum and scattered copy of the counting sort ("Particle
 * worlds, part 3", steps 3-4) and the per-tile index the implementation page
 * builds each substep ("Implementation -- GPU Optimization & Reference
 * Codebases", section 2.1).  The size
 * and layout of a workspace follow from the grid and the particle count; every
 * entry point that is handed a workspace also takes its size in bytes, refuses
 * one that is too small for its own grid and count (MPM_ERR_WORKSPACE), and its
 * kernels compare the stamp the binning left in the workspace with their own
 * arguments before reading anything else (a mismatch is counted in status[3]
 * and the call does nothing, or, for the restricted grid update and clear,
 * falls back to every node). */
int mpm_workspace_bytes(const mpm_grid_desc *grid, int64_t n_particles, size_t *bytes);

/* Offsets of the arrays inside that workspace (host-only; the arrays are
 * those of mpm_ws_layout above, for the same passages). */
int mpm_workspace_layout(const mpm_grid_desc *grid, int64_t n_particles, mpm_ws_layout *layout);

/* Counting sort of the particles into tiles of 4^dim cells by the stencil's
 * base cell ("Particle worlds, part 3", steps 3-4: histogram, exclusive
 * prefix sum, scatter; "Implementation -- GPU Optimization & Reference
 * Codebases", section 2.1: sort + tile).  The caller's arrays are not
 * reordered (section 5 rule 2): the workspace receives the tile histogram
 * and prefix sum, each particle's record index, a binned copy of x, v, C, m
 * (64-byte records, 48 in 2D) tile by tile, and the P2G work items: slices
 * of each tile's records, which mpm_p2g sorts by cell on chip (the cell of a
 * record follows from its position).
 * Particles whose stencil leaves the grid are not binned and
 * are counted in status[0]; particles whose attributes leave the declared
 * ranges are binned as zero-mass records (they contribute nothing, exactly
 * as if skipped) and counted in status[1].  Arrival order inside a tile is
 * not deterministic; the P2G grid built from the bins is (integer sums
 * commute).
 * particles, status: device.  ws: device, ws_bytes >= mpm_workspace_bytes().
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_OVERFLOW (bounds),
 * MPM_ERR_HIP. */
int mpm_bin_particles(const mpm_grid_desc *grid, const mpm_particles *particles, const mpm_ranges *ranges,
                      void *ws, size_t ws_bytes, uint32_t *status, hipStream_t stream);

/* Fixed-point APIC P2G with the quadratic B-spline stencil (3^dim nodes per
 * particle).  For each particle and stencil node, in float32 with one
 * rounding per operation:
 *   wmS = (((m * S) * wx[a]) * wy[b]) * wz[c]
 *   u_d = ((v_d + C_d0 * rx[a]) + C_d1 * ry[b]) + C_d2 * rz[c]
 *   M  += rint(wmS),  P_d += rint(wmS * u_d)     (round to nearest, ties even)
 * where g = x*n, base = floor(g - 1/2), f = g - base, the weights are the
 * quadratic B-spline at distances f, f-1, f-2 and r[o] = (o - f) dx.
 * Sources: "Implementation -- GPU Optimization & Reference Codebases",
 * sections 1 (P2G scatter), 2.1 (fixed-point accumulation, shared-memory
 * tiles, warp-level pre-reduction) and 3.1 (APIC, 3x3 quadratic stencil,
 * affine matrix C); "Mass Matrix Assembly on Tensor Cores for Implicit
 * PIC", shape functions (tensor-product B-spline, stencil placement).
 * Accumulation is in integers, so the grid is identical for every particle
 * order and every scheduling.
 *   bins == NULL: one thread per particle of `particles`, 64-bit global
 *     atomics; skipped particles are counted in status[0]/status[1].
 *   bins != NULL: the workspace (bins_bytes long) filled by
 *     mpm_bin_particles for these particles on this grid with these ranges
 *     (particles->n must be the count binned; its arrays are not read and may
 *     be NULL); one wavefront per work item (a slice of one tile's records)
 *     sorts the slice by cell in LDS, sums each 4 same-cell particles'
 *     contributions in registers, accumulates the tile's node block on chip
 *     and flushes it with one 64-bit atomic per non-zero node and channel.
 *     A workspace whose stamp names another grid, particle count, declared
 *     ranges or a resident binning adds nothing and is counted in status[3].
 * grid: device int64[1+dim][n]^dim, accumulated into (zero it first for a
 * fresh transfer).  The caller must have run mpm_check_bounds on `ranges`;
 * this call re-checks and refuses with MPM_ERR_OVERFLOW.
 * Errors: MPM_ERR_INVALID, MPM_ERR_OVERFLOW, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_p2g(const mpm_grid_desc *grid, const mpm_particles *particles, const mpm_ranges *ranges,
            const void *bins, size_t bins_bytes, int64_t *grid_out, uint32_t *status, hipStream_t stream);

/* Integer-split cloud-in-cell scatter in 2D ("particle to grid transfer in
 * checked integer arithmetic", sections "integers do not care about order"
 * and "the program").  Positions X[2][n] are int32 in units of 1/65536 of a
 * cell on a cells x cells grid; m[n] and vel[2][n] are integers.  Each of
 * q = m, m*vx, m*vy is split along x into far = round(q*fx/65536) (ties to
 * even) and near = q - far, and each part likewise along y, so the four
 * shares sum to q exactly.  grid: device int64[3][cells+1][cells+1],
 * accumulated into.  order (device, may be NULL) gives the visiting order;
 * the result is the same for every order.  Particles outside the grid are
 * skipped and counted in status[0].  The bounds line
 * n * max_mass * max_speed < 2^63 (and max_mass * max_speed * 65536 < 2^63)
 * is checked on the host with the declared maxima.
 * Errors: MPM_ERR_INVALID, MPM_ERR_OVERFLOW, MPM_ERR_HIP. */
int mpm_p2g_cic_split(int64_t n, const int32_t *X, const int32_t *m, const int32_t *vel, const uint32_t *order,
                      int32_t cells, int64_t max_mass, int64_t max_speed, int64_t *grid_out, uint32_t *status,
                      hipStream_t stream);

/* Integer-split quadratic APIC transfer ("particle to grid transfer in
 * checked integer arithmetic", sections "integers do not care about order"
 * and "what is not claimed", which names quadratic weights and the affine
 * term as further splits of the kind the page gives for cloud-in-cell).
 * Positions X[dim][np] are int32 in units of 1/65536 of a cell (node i at
 * i * 65536); m[np], v[dim][np] and C[dim*dim][np] (C_de = C[d*dim+e],
 * velocity per cell) are int64.  With base = floor(x/65536 - 1/2) and
 * F = x - 65536 base per axis, the quadratic B-spline weights are
 * w_0 = (98304 - F)^2 / 2^33, w_2 = (F - 32768)^2 / 2^33, w_1 = 1 - w_0 - w_2
 * and the first moments u_o = w_o (o - F/65536) are u_0 = -(98304 - F)^2 F /
 * 2^49, u_2 = (F - 32768)^2 (131072 - F) / 2^49, u_1 = -u_0 - u_2.  A quantity
 * q is split along an axis into round(q c_0), q minus both outer shares (w)
 * or minus their sum (u), round(q c_2), rounding to nearest with ties to
 * even from the exact 128-bit product; the 3^dim shares are the split along
 * x, then y, then z.  Channel 0 gets the split of m; channel 1+d the split of
 * m v_d plus, for each axis e, the split of m C_de with the first moments on
 * axis e.  Node totals equal particle totals exactly (sum M = sum m,
 * sum P_d = sum m v_d), and the grid is identical for every order.
 * grid: device int64[1+dim][n]^dim (x fastest), accumulated into.  order
 * (device uint32[np], may be NULL) gives the visiting order.  Particles with
 * a node outside [0, n) are skipped and counted in status[0]; particles with
 * |m| > max_mass, |v_d| > max_speed or |C_de| > max_affine are skipped and
 * counted in status[1]; order entries >= np in status[3].  The bounds line
 * np * max_mass * (max_speed + dim * max_affine * 3/2 + 1) < 2^62 is checked
 * on the host (MPM_ERR_OVERFLOW).
 * workspace == NULL: one thread per particle adds each share with a 64-bit
 * global atomic.  workspace != NULL (device, 256-byte aligned, at least
 * mpm_isplit_workspace_bytes): the particles are counting-sorted into
 * 8^dim-cell tiles (a 128-byte copy of each, in tile order, in the
 * workspace) and each slice of up to 2048 particles of a tile
 * accumulates its 10^dim-node block on chip before one atomic per non-zero
 * node and channel.  Both give the same grid.  The workspace is scratch,
 * overwritten by each call; calls sharing one workspace must not overlap.
 * All pointers are device memory owned by the caller; the call is
 * asynchronous on `stream`.
 * Errors: MPM_ERR_INVALID (dim not 2 or 3, n outside [3, 32767], negative
 * maxima, misaligned pointers), MPM_ERR_WORKSPACE, MPM_ERR_OVERFLOW,
 * MPM_ERR_HIP. */
int mpm_p2g_isplit(int32_t dim, int32_t n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                   const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed, int64_t max_affine,
                   void *workspace, size_t workspace_bytes, int64_t *grid_out, uint32_t *status, hipStream_t stream);

/* Bytes of the static device scratch mpm_p2g_isplit_noalloc uses (256 MiB
 * per GPU, held from the library's load until the process ends). */
#define MPM_ISPLIT_SCRATCH_BYTES (256u * 1024u * 1024u)

/* mpm_p2g_isplit's tiled path with its workspace taken from the library's
 * static device scratch instead of the caller's memory: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The call allocates nothing: it
 * makes no hipMalloc/hipFree call and no torch allocation.  Arguments, result,
 * status counters and errors are those of mpm_p2g_isplit with a workspace,
 * and the grid is bit-identical to that call's.  The scratch is one array per
 * GPU (MPM_ISPLIT_SCRATCH_BYTES); every call on a GPU reuses it and clears
 * what must start at zero, so calls that overlap on one GPU (several streams,
 * or host threads without ordering) race and must not be issued.  Inputs
 * whose mpm_isplit_workspace_bytes(dim, n, np) exceeds
 * MPM_ISPLIT_SCRATCH_BYTES are refused with MPM_ERR_SCRATCH before any launch
 * (for example np up to about 2M particles on a 128^3 grid).  The first
 * call on a device looks up that device's copy of the scratch once.
 * Errors: those of mpm_p2g_isplit, MPM_ERR_SCRATCH. */
int mpm_p2g_isplit_noalloc(int32_t dim, int32_t n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                           const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                           int64_t max_affine, int64_t *grid_out, uint32_t *status, hipStream_t stream);

/* Bytes of the workspace mpm_p2g_isplit's tiled path needs for np particles
 * on n^dim nodes (tile counts and starts, each visited particle's rank and
 * its 128-byte tile-ordered record).  Host only.
 * Errors: MPM_ERR_INVALID. */
int mpm_isplit_workspace_bytes(int32_t dim, int32_t n, int64_t np, size_t *bytes);

/* ---- Resident substep: the particle state kept in the binned records ----
 *
 * "Implementation -- GPU Optimization & Reference Codebases", section 2.1:
 * one kernel per tile slice applies the grid update while it loads the
 * tile's node block with its halo, gathers and advects the slice's
 * particles, and scatters them into the next grid through the on-chip block.
 * The state lives in the workspace between substeps; a substep reads grid k
 * and writes grid k+1 (three grid buffers used in turn, each with a byte per
 * 4^dim-node tile that flags the node tiles written into it), and zeroes grid
 * k-1, the one read in the previous substep, once its own items are done, so
 * no clear runs between substeps.  Results are identical to the separate
 * steps (binning, mpm_p2g, mpm_grid_update, mpm_g2p).  A loop:
 *
 *   mpm_bin_resident(ws <- particles); mpm_g2p2g(grid_in = NULL -> A, flags A)
 *   per substep: mpm_g2p2g(A -> B, flags B, clearing C and flags C);
 *                (A, B, C) <- (B, C, A)
 *   to re-bin (particles drift out of their tiles) or to read the state:
 *                mpm_gather_records(ws -> particles), then mpm_bin_resident
 * (With two grids, pass grid_clear = NULL and call mpm_grid_clear_tiles on
 * the grid just read after each substep.)
 */

/* Binning as mpm_bin_particles, keeping every record as it is (no range
 * check: mpm_g2p2g checks the declared ranges at every deposit).  Particles
 * whose stencil leaves the grid are not binned and are counted in status[0].
 * particles, status: device.  ws: device, 256-byte aligned, ws_bytes >=
 * mpm_workspace_bytes(n).  Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE,
 * MPM_ERR_HIP. */
int mpm_bin_resident(const mpm_grid_desc *grid, const mpm_particles *particles, void *ws, size_t ws_bytes,
                     uint32_t *status, hipStream_t stream);

/* One fused substep over the records of a resident binning of n_particles.
 * grid_in != NULL: the grid update of grid_in (as mpm_grid_update: v = P/M
 * + dt g, sticky walls, M = 0 -> 0) feeds the APIC gather and advection of
 * every record (as mpm_g2p, clamps counted in status[2]), written back in
 * place; then the updated records are deposited into grid_out (as mpm_p2g,
 * with the declared ranges checked here: records outside them add nothing
 * and are counted in status[1]).  grid_in is only read.  grid_in == NULL: the
 * records are deposited as they are.  Records that left their tile since the
 * binning deposit with global atomics, so the result does not depend on
 * when the caller re-bins.  grid_out must be zero on entry; every node tile
 * it writes is flagged (set to 1) in tiles_out, uint8[(n/4)^dim], for
 * mpm_grid_clear_tiles.  grid_clear != NULL: a third grid, neither grid_in
 * nor grid_out, whose node tiles flagged in tiles_clear (not tiles_out) are
 * zeroed in every channel, and those flags reset, as mpm_grid_clear_tiles
 * would (grid_clear == NULL: tiles_clear is ignored).  All pointers device;
 * ws is ws_bytes long.  A workspace whose stamp names another grid or
 * particle count does nothing and is counted in status[3].
 * Errors: MPM_ERR_INVALID, MPM_ERR_OVERFLOW (bounds for n_particles and the
 * ranges, as mpm_check_bounds), MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_g2p2g(const mpm_grid_desc *grid, const mpm_ranges *ranges, void *ws, size_t ws_bytes, int64_t n_particles,
              const int64_t *grid_in, int64_t *grid_out, uint8_t *tiles_out, int64_t *grid_clear,
              uint8_t *tiles_clear, float dt, const float *gravity, int32_t sticky, uint32_t *status,
              hipStream_t stream);

/* Zeroes every node of the node tiles flagged in tiles (uint8[(n/4)^dim]),
 * in every channel of grid, then clears the flags.  Errors: MPM_ERR_INVALID,
 * MPM_ERR_HIP. */
int mpm_grid_clear_tiles(const mpm_grid_desc *grid, int64_t *grid_io, uint8_t *tiles, hipStream_t stream);

/* The resident substep split in three launches instead of the fused kernel's
 * one ("Implementation -- GPU Optimization & Reference Codebases", section
 * 2.1: the transfer cycle over the binned state; the node tiles a deposit
 * wrote are the ones the next update touches):
 *
 *   mpm_bin_resident(ws <- particles); mpm_g2p2g(grid_in = NULL -> A, flags A)
 *   per substep: mpm_grid_update_tiles(A, flags A -> vg)      (A zeroed)
 *                mpm_g2p_records(vg, records in place)
 *                mpm_g2p2g(grid_in = NULL -> B, flags B)      (the deposit)
 *                (A, B) <- (B, A)
 *
 * Results are identical to the fused kernel's and to the separate steps'.
 * Two grids suffice: the update consumes the grid it reads. */

/* Grid update of the node tiles flagged in tiles (uint8[(n/4)^dim], as
 * mpm_g2p2g writes them): at every node of a flagged tile, v = P/M + dt g
 * (M != 0), 0 where M == 0 and on the sticky walls, into vg; M and P set to
 * zero; then every flag reset.  Nodes of unflagged tiles are not touched
 * (their vg stays as it was).  Same arithmetic as mpm_grid_update.  All
 * pointers device.  Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_grid_update_tiles(const mpm_grid_desc *grid, int64_t *grid_io, uint8_t *tiles, float *vg, float dt,
                          const float *gravity, int32_t sticky, hipStream_t stream);

/* The APIC gather and advection (as mpm_g2p: vg read, clamps counted in
 * status[2]) of every record of a resident binning of n_particles, written
 * back into the record in place (x, v, C; m kept), records visited in tile
 * order.  ws: device, ws_bytes long; a workspace whose stamp names another
 * grid or particle count does nothing and is counted in status[3].
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_g2p_records(const mpm_grid_desc *grid, void *ws, size_t ws_bytes, int64_t n_particles, const float *vg,
                    float dt, uint32_t *status, hipStream_t stream);

/* Copies x, v and C of every binned particle from its record back to the
 * caller's arrays (particles->n must be the count the workspace was binned
 * with; m and particles that were not binned are left as they are).  ws is
 * ws_bytes long; a workspace whose stamp names another grid or particle count
 * copies nothing and is counted in status[3].
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_gather_records(const mpm_grid_desc *grid, const void *ws, size_t ws_bytes, const mpm_particles *particles,
                       uint32_t *status, hipStream_t stream);

/* Grid update with consume-and-zero ("Implementation -- GPU Optimization &
 * Reference Codebases", section 1 four-phase step; section 2.1 and rule 4
 * of section 5: each accumulator has one reader, which zeroes it; rule 1:
 * convert the fixed-point sums once, here; rule 7: gravity belongs to the
 * solver).  Per node: where M != 0, v_d = (float)((double)P_d / (double)M)
 * then v_d = v_d + (dt * g_d) (the product formed once in float32); where
 * M == 0, v = 0; nodes within `sticky` nodes of any face get v = 0; then
 * M and P are set to 0.
 * bins == NULL: every node.  bins != NULL: the workspace (bins_bytes long,
 * at least its particle-count-independent prefix) of the mpm_bin_particles
 * call whose P2G filled the grid (same grid descriptor; bins stamped for
 * another grid fall back to every node);
 * only the nodes of 4^dim-node tiles that this P2G can reach (tiles whose
 * own or lower-neighbour cell tiles hold binned particles) are updated, and
 * vg elsewhere is left as it was.  Every other accumulator is already zero
 * when the grid was zero before that P2G, and G2P of the same particles reads
 * vg only at reachable nodes, so a substep loop gives the same particles as
 * with every node updated.  The call writes the tile_active flags of the
 * workspace.
 * grid: device int64[1+dim][n]^dim, read and zeroed.  vg: device
 * float[dim][n]^dim, written.  gravity: host float[dim].
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_grid_update(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, float *vg, float dt,
                    const float *gravity, int32_t sticky, hipStream_t stream);

/* Accumulator reset before a P2G ("Implementation -- GPU Optimization &
 * Reference Codebases", section 2.1 and rule 4 of section 5: accumulators
 * must start each step at zero; sparse grids reset only the blocks in use).
 * bins == NULL: every channel of every node is set to 0.  bins != NULL: the
 * workspace (bins_bytes long, as for mpm_grid_update) of the
 * mpm_bin_particles call whose P2G last added to this grid (same grid
 * descriptor; bins stamped for another grid fall back to every node); only
 * the nodes of the 4^dim-node tiles that this
 * P2G could reach are zeroed (the set mpm_grid_update restricts itself to),
 * which zeroes the whole grid when it was zero before that P2G.  The call
 * writes the tile_active flags of the workspace.
 * grid: device int64[1+dim][n]^dim, written.
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_grid_clear(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, hipStream_t stream);

/* APIC grid-to-particle gather and advection ("Implementation -- GPU
 * Optimization & Reference Codebases", sections 1 and 3.1).  Per particle,
 * over its stencil nodes in lexicographic order (x offset outermost), with
 * w = (wx[a] * wy[b]) * wz[c] and wv_d = w * vg_d, the per-axis offset sums
 * S_de[o] += wv_d (o the node's offset along axis e); then
 * v_d = (S_d0[0] + S_d0[1]) + S_d0[2],
 * B_de = (r_e[0] S_de[0] + r_e[1] S_de[1]) + r_e[2] S_de[2],
 * C = B * (4 n^2), x_e += dt * v_e, and x_e is
 * clamped to [dx, (n-2) dx] (clamped particles counted in status[2]).
 * Particles whose stencil leaves the grid are left unchanged and counted in
 * status[0].  particles: device, x, v, C read/written in place (m unused).
 * vg: device float[dim][n]^dim.
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_g2p(const mpm_grid_desc *grid, const float *vg, const mpm_particles *particles, float dt,
            uint32_t *status, hipStream_t stream);

/* MLS-MPM stress term of a Neo-Hookean solid ("Implementation -- GPU
 * Optimization & Reference Codebases", section 3.1, part 2 of the guide
 * described there: P = mu (F - F^-T) + lambda log(J) F^-T, J = det F,
 * sigma = P F^T / J).  The stress enters P2G through the affine term
 * Q = m C - dt vol sigma 4 n^2 (vol sigma = vol0 P F^T); divided by m, the
 * APIC P2G is unchanged when its affine matrix is
 *   C' = C - (dt vol0 4 n^2 / m) P F^T,
 * which this call writes to C_out, for binning and P2G to read in place of C.
 * Per particle in float64 in this order: the cofactor matrix cof of F (F^-T =
 * cof / J), J = (F00 cof00 + F01 cof01) + F02 cof02 (2D: F00 F11 - F01 F10),
 * P_de = mu (F_de - cof_de / J) + (lambda log J) (cof_de / J),
 * tau_de = sum_q P_dq F_eq, k = ((dt vol0) 4 n^2) / m, C'_de = C_de - k tau_de
 * rounded to float32 once.  Particles with det F <= 0 (counted in status[0])
 * or m == 0 get C' = C.
 * particles: device; C and m read (x, v unused).  F: device float[dim*dim][n]
 * component-major like C.  vol0: device float[n], initial volumes.  C_out:
 * device float[dim*dim][n], written (may not alias C).
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_neohookean_affine(const mpm_grid_desc *grid, const mpm_particles *particles, const float *F, const float *vol0,
                          float dt, float mu, float lambda, float *C_out, uint32_t *status, hipStream_t stream);

/* Deformation gradient update after G2P (the same part of the guide):
 * F <- (I + dt C) F with C the particles' new affine matrices, in float32:
 * G_dq = [d == q] + dt C_dq, F'_de = (G_d0 F_0e + G_d1 F_1e) + G_d2 F_2e.
 * particles: device, C read.  F: device float[dim*dim][n], read and written.
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_update_deformation(const mpm_grid_desc *grid, const mpm_particles *particles, float *F, float dt,
                           hipStream_t stream);

/* The two per-particle passes of the same part of the guide that sit between
 * one substep's G2P and the next substep's binning, in one pass: F is updated
 * exactly as mpm_update_deformation does, then C_out receives C' exactly as
 * mpm_neohookean_affine computes it from the updated F and the particles' C
 * (the same float32 and float64 operations in the same order, so the results
 * are bit-identical to those two calls in sequence; C, F, m and vol0 are read
 * once).  dt is the substep's time step, used for both.
 * particles: device; C and m read.  F: device float[dim*dim][n], read and
 * written.  vol0: device float[n].  C_out: device float[dim*dim][n], written
 * (may alias neither C nor F).  status[0] counts particles whose updated F
 * has det <= 0 (their C' = C).
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_update_deformation_stress(const mpm_grid_desc *grid, const mpm_particles *particles, float *F,
                                  const float *vol0, float dt, float mu, float lambda, float *C_out, uint32_t *status,
                                  hipStream_t stream);

/* The elastic substep's G2P and the pass after it, in one launch: exactly
 * mpm_g2p (the gather and advection from vg, with dt) followed by
 * mpm_update_deformation_stress (F updated with the new C, then C_out = C' of
 * the next substep from the updated F), the same operations in the same
 * order, so the results and the status counts are bit-identical to those two
 * calls in sequence.  The gather runs over the particles first and the second
 * pass reads back the C it wrote.
 * vg: device float[dim][nodes].  particles: device; x, v, C read and written,
 * m read.  F: device float[dim*dim][n], read and written.  vol0: device
 * float[n].  C_out: device float[dim*dim][n], written (may alias neither C nor
 * F).  status[0] counts particles outside the grid and particles whose
 * updated F has det <= 0, status[2] clamped particles.
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_g2p_update_deformation_stress(const mpm_grid_desc *grid, const float *vg, const mpm_particles *particles,
                                      float dt, float *F, const float *vol0, float mu, float lambda, float *C_out,
                                      uint32_t *status, hipStream_t stream);

/* ---- Position-based MPM (PB-MPM): the iteration loop for an elastic material ----
 *
 * "Implementation -- GPU Optimization & Reference Codebases", section 3.3.2.
 * A particle carries its displacement over the substep d (in particles->v)
 * and its displacement gradient D (in particles->C, same layout), with x, m
 * and the deformation gradient F (float[dim*dim][n], like C).  A substep:
 *
 *   repeat `iterations` times (the page's default 5):
 *     mpm_pbmpm_project_elastic     D toward the elastic target
 *     mpm_bin_particles, mpm_p2g    mass and momentum m (d + D (x_i - x_p)),
 *                                   no stress term
 *     mpm_pbmpm_grid_update         mass-normalise, guardian
 *     mpm_g2p with dt = 0           gather d and D (x stays in place)
 *   mpm_pbmpm_integrate             x += d, gravity into the next d
 *   mpm_update_deformation, dt = 1  F <- (I + D) F
 *
 * d and D carry over to the next substep as its starting guess (warm start).
 * Every iteration's G2P but the last may run together with the next
 * iteration's projection (mpm_pbmpm_g2p_project, or _records to skip the
 * re-binning), and the last with the integrate step and the F update
 * (mpm_pbmpm_g2p_integrate), the same results in fewer passes.
 */

/* particleUpdate for an elastic material: the target shape is a rotation, the
 * polar rotation R of the trial deformation Ft = (I + D) F (Newton's iteration
 * R <- (R + R^-T) / 2 from R = Ft, polar_iters steps, in place of an SVD); the
 * displacement gradient reaching it is D* = R F^-1 - I, and D relaxes toward it:
 * D <- D + relax (D* - D) (relax in [0, 2]; the page's default 1.5 over-relaxes).
 * In float64 in this order, D rounded to float32 once:
 *   Ft_de = sum_q ([d == q] + D_dq) F_qe, R_de <- (R_de + cof(R)_de / det R) / 2,
 *   F^-1_qe = cof(F)_eq / det F, D*_de = sum_q R_dq F^-1_qe - [d == e],
 *   D_de <- D_de + relax (D*_de - D_de),
 * cof the cofactor matrix (det = (a00 cof00 + a01 cof01) + a02 cof02).
 * Particles whose Ft, F or a Newton iterate has det <= 0 keep D and are
 * counted in status[0].  particles: device; C (= D) read and written, x, v, m
 * unused.  F: device float[dim*dim][n].  polar_iters in [0, 64].
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_pbmpm_project_elastic(const mpm_grid_desc *grid, const mpm_particles *particles, const float *F, float relax,
                              int32_t polar_iters, uint32_t *status, hipStream_t stream);

/* The loop's G2P gather of one iteration and the elastic projection that
 * opens the next, in one pass: exactly mpm_g2p with dt = 0 (d and D gathered
 * from dg, x kept and clamped as there) followed by mpm_pbmpm_project_elastic
 * on the D it gathered (or on the stored D of a particle outside the grid,
 * which the gather skips); the same operations in the same order, so the
 * results and the status counts are bit-identical to those two calls in
 * sequence.  A substep then runs mpm_pbmpm_project_elastic once before its
 * first iteration and this call after every iteration but the last, whose
 * G2P is mpm_g2p.
 * dg: device float[dim][nodes], the displacement grid of mpm_pbmpm_grid_update.
 * particles: device; x read (and clamped), v (d) written, C (D) read and
 * written.  F: device float[dim*dim][n].  relax in [0, 2], polar_iters in
 * [0, 64].  status[0] counts particles outside the grid and refused
 * projections, status[2] clamps.
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_pbmpm_g2p_project(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles, const float *F,
                          float relax, int32_t polar_iters, uint32_t *status, hipStream_t stream);

/* mpm_pbmpm_g2p_project, and then each particle's record in ws rewritten from
 * its new state exactly as mpm_bin_particles writes it (x, v = d, C = D, m;
 * v, C and m zeroed and counted in status[1] when outside the ranges), so that
 * the next iteration's mpm_p2g runs on the same binning: the particles' x
 * moves only by the gather's clamp to [dx, (n - 2) dx], which keeps each one in
 * its cell (x n is exact for a power-of-two n, and the clamp maps x n in
 * [1/2, 1) to 1 and in (n - 2, n - 3/2) to n - 2, each with its stencil base),
 * so the tiles, work items and slots stay valid.  The P2G grid is then
 * bit-identical to the one after a fresh binning (its integer sums do not
 * depend on the records' order inside a tile).  A substep bins once, after its
 * first projection, and calls this after every iteration but the last.
 * ws, ws_bytes: the workspace of mpm_bin_particles on these particles with the
 * same grid and ranges, binned since x last changed outside these calls; a
 * workspace binned for another grid, particle count or ranges is refused on
 * the device (nothing is written, status[3] incremented).  particles: as for
 * mpm_pbmpm_g2p_project, and m read.  Other arguments and status counts as for
 * mpm_pbmpm_g2p_project.
 * Errors: MPM_ERR_INVALID, MPM_ERR_OVERFLOW, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_pbmpm_g2p_project_records(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles,
                                  const float *F, float relax, int32_t polar_iters, const mpm_ranges *ranges, void *ws,
                                  size_t ws_bytes, uint32_t *status, hipStream_t stream);

/* The loop's last G2P gather and the end of the substep in one launch:
 * exactly mpm_g2p with dt = 0 on dg (d and D gathered, x kept and clamped),
 * then mpm_pbmpm_integrate (x += d clamped, d += g dt^2) and
 * mpm_update_deformation with dt = 1 (F <- (I + D) F), the same operations in
 * the same order, so the results and the status counts are bit-identical to
 * those three calls in sequence.  A substep then ends with this call in place
 * of its last mpm_g2p.
 * dg: device float[dim][nodes].  particles: device; x, v (d) and C (D) read
 * and written.  F: device float[dim*dim][n], read and written.  gravity: host
 * float[dim].  status[0] counts particles outside the grid, status[2] clamps
 * (by the gather and by the integrate step).
 * Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_pbmpm_g2p_integrate(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles, float *F,
                            float dt, const float *gravity, uint32_t *status, hipStream_t stream);

/* gridUpdate in displacement form (the same section: mass-normalise, then the
 * guardian projects each node's displaced position back into bounds).  Per
 * node: where M != 0, d_e = (float)((double)P_e / (double)M), then with the
 * node's position X_e = i_e dx, d_e = fminf(fmaxf(X_e + d_e, lo), hi) - X_e,
 * lo = band dx, hi = (n - 1 - band) dx; d = 0 where M == 0; then M = P = 0.  No
 * gravity (mpm_pbmpm_integrate puts it into the next displacement).  bins and
 * bins_bytes as for mpm_grid_update (NULL: every node; else only the node
 * tiles the binned P2G can reach).  grid: device int64[1+dim][n]^dim, read and
 * zeroed.  dg: device float[dim][n]^dim, written.  band in [1, (n - 2) / 2].
 * Errors: MPM_ERR_INVALID, MPM_ERR_WORKSPACE, MPM_ERR_HIP. */
int mpm_pbmpm_grid_update(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, float *dg,
                          int32_t band, hipStream_t stream);

/* particleIntegrate for an elastic material (the same section), without the
 * deformation update (mpm_update_deformation with dt = 1): per particle
 * x_e <- x_e + d_e (float32), clamped to [dx, (n - 2) dx] with clamped
 * particles counted in status[2]; then d_e <- d_e + g_e * (dt * dt) (the
 * product formed once in float32): gravity goes into the next substep's
 * displacement.  particles: device, x and v (= d) read and written.
 * gravity: host float[dim].  Errors: MPM_ERR_INVALID, MPM_ERR_HIP. */
int mpm_pbmpm_integrate(const mpm_grid_desc *grid, const mpm_particles *particles, float dt, const float *gravity,
                        uint32_t *status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MPM_H */
