// abi.hip -- the extern "C" entry points of libmpm: argument validation, the
// host-side bounds line, workspace layout, and launches on the caller's stream.
#include <math.h>
#include <string.h>

#include <atomic>

#include "resident.hpp"
#include "pbmpm_device.hpp"
#include "stress.hpp"

namespace mpmk {

int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace mpmk

namespace {

using namespace mpmk;

// Record indices and tile ranks are uint32.
constexpr int64_t kMaxParticles = 0xFFFFFFF0;

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void *p, size_t a) { return p != nullptr && ((uintptr_t)p % a) == 0; }

int check_desc(const mpm_grid_desc *g)
{
    if (!g || (g->dim != 2 && g->dim != 3))
        return MPM_ERR_INVALID;
    const int nmax = g->dim == 3 ? 512 : 1024;
    if (!is_pow2(g->n) || g->n < 8 || g->n > nmax)
        return MPM_ERR_INVALID;
    if (g->frac_bits < 0 || g->frac_bits > 60 || g->tile != kTile)
        return MPM_ERR_INVALID;
    return MPM_OK;
}

int check_ranges(const mpm_ranges *r)
{
    if (!r)
        return MPM_ERR_INVALID;
    if (!(r->max_mass >= 0.0) || !(r->max_speed >= 0.0) || !(r->max_affine >= 0.0))
        return MPM_ERR_INVALID;
    return MPM_OK;
}

// Largest float not above v (v >= 0), so |x| <= result in float32 decides
// exactly |x| <= v in real numbers for every float x.
float floor_to_float(double v)
{
    float f = (float)v;
    if ((double)f > v)
        f = nextafterf(f, -INFINITY);
    return f;
}

RangesF ranges_f(const mpm_ranges *r)
{
    RangesF o;
    o.max_mass = floor_to_float(r->max_mass);
    o.max_speed = floor_to_float(r->max_speed);
    o.max_affine = floor_to_float(r->max_affine);
    return o;
}

// log2 of the largest quantised contribution under the declared ranges.
double log2_max_contribution(const mpm_grid_desc *g, const mpm_ranges *r)
{
    const double dx = 1.0 / (double)g->n;
    const double wmax = g->dim == 3 ? 27.0 / 64.0 : 9.0 / 16.0;     // (3/4)^dim
    double umax = r->max_speed + (double)g->dim * r->max_affine * 1.5 * dx;
    if (umax < 1.0)
        umax = 1.0;                                                   // mass channel: u = 1
    const double q = ldexp(1.0, g->frac_bits) * wmax * r->max_mass * umax * (1.0 + ldexp(1.0, -20)) + 1.0;
    return log2(q);
}

struct Layout {
    mpm_ws_layout l;
};

int64_t pow_int(int64_t b, int e)
{
    int64_t r = 1;
    for (int i = 0; i < e; ++i)
        r *= b;
    return r;
}

void make_layout(const mpm_grid_desc *g, int64_t np, mpm_ws_layout *o)
{
    memset(o, 0, sizeof(*o));
    const int64_t n_cells = pow_int(g->n, g->dim);
    const int64_t n_tiles = pow_int(g->n / kTile, g->dim);
    const int64_t busy = np < n_tiles ? (np > 0 ? np : 1) : n_tiles;       // tiles that can hold particles
    // work items: every non-empty tile's records cut into slices, all full
    // but the last
    const int64_t slice = g->dim == 3 ? slice_records<3>() : slice_records<2>();
    const int64_t max_items = np / slice + busy;
    const int64_t n_fields = g->dim == 3 ? rec_floats<3>() : rec_floats<2>();
    const int64_t plan_blocks = (n_tiles + kPlanTiles - 1) / kPlanTiles;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t u4 = sizeof(uint32_t);
    const int64_t n1 = np > 0 ? np : 1;
    o->tile_count = take(u4 * (size_t)n_tiles);
    o->tile_start = take(u4 * (size_t)(n_tiles + 1));
    o->tile_active = take((size_t)n_tiles);
    o->meta = take(u4 * kMetaWords);                 // (offsets up to here do not depend on np)
    o->items = take(u4 * 4 * (size_t)max_items);
    o->rank = take(u4 * (size_t)n1);
    o->slot = take(u4 * (size_t)n1);
    o->cell_key = take((size_t)n1 + 4);
    o->sorted = take(sizeof(float) * (size_t)(n_fields * n1));
    o->scan_tmp = take(u4 * (size_t)(kPlanStride * plan_blocks));
    o->n_cells = n_cells;
    o->n_tiles = n_tiles;
    o->max_items = max_items;
    o->n_fields = n_fields;
    o->rows_per_item = kRowsPerItem;
    o->total_bytes = off;
}

// Bytes of the workspace prefix whose offsets do not depend on the particle
// count (tile arrays and meta): what the grid update and clear read.
size_t fixed_prefix_bytes(const mpm_grid_desc *g)
{
    mpm_ws_layout l;
    make_layout(g, 0, &l);
    return l.meta + sizeof(uint32_t) * kMetaWords;
}

uint32_t float_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

BinStamp make_stamp(const mpm_grid_desc *g, int64_t np, RangesF r, bool keep)
{
    BinStamp s;
    s.magic = kStampMagic;
    s.dim = (uint32_t)g->dim;
    s.n = (uint32_t)g->n;
    s.np_lo = (uint32_t)((uint64_t)np & 0xFFFFFFFFu);
    s.np_hi = (uint32_t)((uint64_t)np >> 32);
    s.max_mass = keep ? 0u : float_bits(r.max_mass);
    s.max_speed = keep ? 0u : float_bits(r.max_speed);
    s.max_affine = keep ? 0u : float_bits(r.max_affine);
    s.keep = keep ? 1u : 0u;
    return s;
}

BinView bin_view(void *ws, const mpm_ws_layout &l, const BinStamp &stamp)
{
    char *b = (char *)ws;
    BinView v;
    v.stamp = stamp;
    v.tile_count = (uint32_t *)(b + l.tile_count);
    v.tile_start = (uint32_t *)(b + l.tile_start);
    v.items = (uint32_t *)(b + l.items);
    v.meta = (uint32_t *)(b + l.meta);
    v.rank = (uint32_t *)(b + l.rank);
    v.slot = (uint32_t *)(b + l.slot);
    v.cell_key = (uint8_t *)(b + l.cell_key);
    v.sorted = (float *)(b + l.sorted);
    v.tile_active = (uint8_t *)(b + l.tile_active);
    v.scan_tmp = (uint32_t *)(b + l.scan_tmp);
    v.n_cells = l.n_cells;
    v.n_tiles = l.n_tiles;
    v.max_items = l.max_items;
    v.n_fields = l.n_fields;
    return v;
}

int check_particles(const mpm_grid_desc *g, const mpm_particles *p, bool need_arrays, bool need_mass)
{
    if (!p || p->n < 0 || p->n > kMaxParticles)
        return MPM_ERR_INVALID;
    if (!need_arrays || p->n == 0)
        return MPM_OK;
    if (!aligned(p->x, 4) || !aligned(p->v, 4))
        return MPM_ERR_INVALID;
    if (p->C && !aligned(p->C, 4))
        return MPM_ERR_INVALID;
    if (need_mass && !aligned(p->m, 4))
        return MPM_ERR_INVALID;
    (void)g;
    return MPM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MPM_OK : MPM_ERR_HIP; }

}  // namespace

extern "C" {

const char *mpm_version(void) { return "libmpm 0.1.0 gfx950"; }

const char *mpm_strerror(int code)
{
    switch (code) {
    case MPM_OK: return "ok";
    case MPM_ERR_INVALID: return "invalid argument (descriptor, pointer, alignment or size)";
    case MPM_ERR_OVERFLOW: return "declared ranges could overflow the fixed-point accumulators";
    case MPM_ERR_DOMAIN: return "particle outside the grid";
    case MPM_ERR_WORKSPACE: return "workspace too small";
    case MPM_ERR_HIP: return "HIP runtime or launch failure";
    case MPM_ERR_SCRATCH: return "input needs more than the static scratch holds (MPM_ISPLIT_SCRATCH_BYTES)";
    default: return "unknown error";
    }
}

int mpm_check_bounds(const mpm_grid_desc *grid, int64_t n_particles, const mpm_ranges *ranges, double *log2_bound)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_ranges(ranges)) != MPM_OK || n_particles < 0)
        return rc != MPM_OK ? rc : MPM_ERR_INVALID;
    const double lq = log2_max_contribution(grid, ranges);
    const double lb = lq + log2((double)(n_particles > 0 ? n_particles : 1));
    if (log2_bound)
        *log2_bound = lb;
    // int64 node sums over all particles; exact float64 partial sums over one
    // work item (at most kRowsPerItem * kRowSlots particles) on chip.
    if (!(lb < 62.999) || !(lq + log2((double)(kRowsPerItem * kRowSlots)) < 53.0))
        return MPM_ERR_OVERFLOW;
    return MPM_OK;
}

int mpm_workspace_layout(const mpm_grid_desc *grid, int64_t n_particles, mpm_ws_layout *layout)
{
    if (check_desc(grid) != MPM_OK || n_particles < 0 || n_particles > kMaxParticles || !layout)
        return MPM_ERR_INVALID;
    make_layout(grid, n_particles, layout);
    return MPM_OK;
}

int mpm_workspace_bytes(const mpm_grid_desc *grid, int64_t n_particles, size_t *bytes)
{
    mpm_ws_layout l;
    const int rc = mpm_workspace_layout(grid, n_particles, &l);
    if (rc != MPM_OK || !bytes)
        return rc != MPM_OK ? rc : MPM_ERR_INVALID;
    *bytes = l.total_bytes;
    return MPM_OK;
}

int mpm_bin_particles(const mpm_grid_desc *grid, const mpm_particles *particles, const mpm_ranges *ranges, void *ws,
                      size_t ws_bytes, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_ranges(ranges)) != MPM_OK ||
        (rc = check_particles(grid, particles, true, true)) != MPM_OK)
        return rc;
    if (!aligned(ws, 256) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    if ((rc = mpm_check_bounds(grid, particles->n, ranges, nullptr)) != MPM_OK)
        return rc;
    mpm_ws_layout l;
    make_layout(grid, particles->n, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const RangesF rf = ranges_f(ranges);
    const BinView b = bin_view(ws, l, make_stamp(grid, particles->n, rf, false));
    Fields f{ particles->x, particles->v, particles->C, particles->m, particles->n };
    return hip_status(launch_bin(grid->dim, grid->n, f, rf, b, status, stream));
}

int mpm_bin_resident(const mpm_grid_desc *grid, const mpm_particles *particles, void *ws, size_t ws_bytes,
                     uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, true)) != MPM_OK)
        return rc;
    if (!aligned(ws, 256) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    mpm_ws_layout l;
    make_layout(grid, particles->n, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    const BinView b = bin_view(ws, l, make_stamp(grid, particles->n, none, true));
    Fields f{ particles->x, particles->v, particles->C, particles->m, particles->n };
    return hip_status(launch_bin(grid->dim, grid->n, f, none, b, status, stream, true));
}

int mpm_g2p2g(const mpm_grid_desc *grid, const mpm_ranges *ranges, void *ws, size_t ws_bytes, int64_t n_particles,
              const int64_t *grid_in, int64_t *grid_out, uint8_t *tiles_out, int64_t *grid_clear,
              uint8_t *tiles_clear, float dt, const float *gravity, int32_t sticky, uint32_t *status,
              hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_ranges(ranges)) != MPM_OK)
        return rc;
    if (n_particles < 0 || n_particles > kMaxParticles || !aligned(ws, 256) || !aligned(grid_out, 8) ||
        !aligned(tiles_out, 4) || !aligned(status, 4) || (grid_in && !aligned(grid_in, 8)) || grid_in == grid_out)
        return MPM_ERR_INVALID;
    if (grid_clear && (!aligned(grid_clear, 8) || !aligned(tiles_clear, 4) || grid_clear == grid_out ||
                       grid_clear == grid_in || tiles_clear == tiles_out))
        return MPM_ERR_INVALID;
    if (grid_in && (!gravity || sticky < 0 || sticky > grid->n / 2 || !(dt >= 0.0f)))
        return MPM_ERR_INVALID;
    if ((rc = mpm_check_bounds(grid, n_particles, ranges, nullptr)) != MPM_OK)
        return rc;
    mpm_ws_layout l;
    make_layout(grid, n_particles, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const float g3[3] = { gravity ? gravity[0] : 0.0f, gravity ? gravity[1] : 0.0f,
                          gravity && grid->dim == 3 ? gravity[2] : 0.0f };
    const RangesF rf = ranges_f(ranges);
    const BinView b = bin_view(ws, l, make_stamp(grid, n_particles, rf, true));
    return hip_status(launch_g2p2g(grid->dim, grid->n, grid->frac_bits, b, rf, grid_in,
                                   grid_out, tiles_out, grid_clear, grid_clear ? tiles_clear : nullptr, dt, g3, sticky,
                                   status, stream));
}

int mpm_grid_clear_tiles(const mpm_grid_desc *grid, int64_t *grid_io, uint8_t *tiles, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !aligned(grid_io, 8) || !aligned(tiles, 4))
        return MPM_ERR_INVALID;
    return hip_status(launch_grid_clear_tiles(grid->dim, grid->n, grid_io, tiles, stream));
}

int mpm_grid_update_tiles(const mpm_grid_desc *grid, int64_t *grid_io, uint8_t *tiles, float *vg, float dt,
                          const float *gravity, int32_t sticky, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !aligned(grid_io, 8) || !aligned(tiles, 4) || !aligned(vg, 4) || !gravity ||
        sticky < 0 || sticky > grid->n / 2 || !(dt >= 0.0f))
        return MPM_ERR_INVALID;
    return hip_status(launch_grid_update_tiles(grid->dim, grid->n, grid_io, tiles, vg, dt, gravity, sticky, stream));
}

int mpm_g2p_records(const mpm_grid_desc *grid, void *ws, size_t ws_bytes, int64_t n_particles, const float *vg,
                    float dt, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK)
        return rc;
    if (n_particles < 0 || n_particles > kMaxParticles || !aligned(ws, 256) || !aligned(vg, 4) ||
        !aligned(status, 4) || !(dt >= 0.0f))
        return MPM_ERR_INVALID;
    mpm_ws_layout l;
    make_layout(grid, n_particles, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    return hip_status(launch_g2p_records(grid->dim, grid->n, bin_view(ws, l, make_stamp(grid, n_particles, none, true)),
                                         vg, dt, status, stream));
}

int mpm_gather_records(const mpm_grid_desc *grid, const void *ws, size_t ws_bytes, const mpm_particles *particles,
                       uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, false)) != MPM_OK)
        return rc;
    if (!aligned(ws, 256) || !aligned(status, 4) || (particles->n > 0 && !particles->C))
        return MPM_ERR_INVALID;
    mpm_ws_layout l;
    make_layout(grid, particles->n, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    return hip_status(launch_gather_records(grid->dim, particles->n,
                                            bin_view((void *)ws, l, make_stamp(grid, particles->n, none, true)),
                                            particles->x, particles->v, particles->C, status, stream));
}

int mpm_p2g(const mpm_grid_desc *grid, const mpm_particles *particles, const mpm_ranges *ranges, const void *bins,
            size_t bins_bytes, int64_t *grid_out, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_ranges(ranges)) != MPM_OK ||
        (rc = check_particles(grid, particles, bins == nullptr, true)) != MPM_OK)
        return rc;
    if (!aligned(grid_out, 8) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    if ((rc = mpm_check_bounds(grid, particles->n, ranges, nullptr)) != MPM_OK)
        return rc;
    if (bins) {
        if (!aligned(bins, 256))
            return MPM_ERR_INVALID;
        mpm_ws_layout l;
        make_layout(grid, particles->n, &l);
        if (bins_bytes < l.total_bytes)
            return MPM_ERR_WORKSPACE;
        const BinView b = bin_view((void *)bins, l, make_stamp(grid, particles->n, ranges_f(ranges), false));
        return hip_status(launch_p2g_tiled(grid->dim, grid->n, grid->frac_bits, b, grid_out, status, stream));
    }
    Fields f{ particles->x, particles->v, particles->C, particles->m, particles->n };
    return hip_status(launch_p2g_direct(grid->dim, grid->n, grid->frac_bits, f, nullptr, ranges_f(ranges), grid_out,
                                        status, stream));
}

int mpm_p2g_cic_split(int64_t n, const int32_t *X, const int32_t *m, const int32_t *vel, const uint32_t *order,
                      int32_t cells, int64_t max_mass, int64_t max_speed, int64_t *grid_out, uint32_t *status,
                      hipStream_t stream)
{
    if (n < 0 || n > (int64_t)0xFFFFFFF0 || cells < 1 || cells > 32767 || max_mass < 0 || max_speed < 0)
        return MPM_ERR_INVALID;
    if (!aligned(grid_out, 8) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    if (n > 0 && (!aligned(X, 4) || !aligned(m, 4) || !aligned(vel, 4) || (order && !aligned(order, 4))))
        return MPM_ERR_INVALID;
    // bounds line: n * max_mass * max_speed and the split products q * f fit int64
    const long double sp = (long double)(max_speed > 1 ? max_speed : 1);
    const long double lim = 9223372036854775807.0L;
    if ((long double)n * (long double)max_mass * sp > lim || (long double)max_mass * sp * 65536.0L > lim)
        return MPM_ERR_OVERFLOW;
    return hip_status(launch_p2g_cic_split(n, X, m, vel, order, cells, grid_out, status, stream));
}

int mpm_isplit_workspace_bytes(int32_t dim, int32_t n, int64_t np, size_t *bytes)
{
    if ((dim != 2 && dim != 3) || n < 3 || n > 32767 || np < 0 || np > (int64_t)0xFFFFFFF0 || !bytes)
        return MPM_ERR_INVALID;
    *bytes = isplit_layout(dim, n, np).total;
    return MPM_OK;
}

}  // extern "C"

namespace {

// Arguments and bounds line of the integer-split transfer (both entry points).
int check_isplit(int32_t dim, int32_t n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                 const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed, int64_t max_affine,
                 const int64_t *grid_out, const uint32_t *status)
{
    if ((dim != 2 && dim != 3) || n < 3 || n > 32767 || np < 0 || np > (int64_t)0xFFFFFFF0 || max_mass < 0 ||
        max_speed < 0 || max_affine < 0)
        return MPM_ERR_INVALID;
    if (!aligned(grid_out, 8) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    if (np > 0 && (!aligned(X, 4) || !aligned(m, 8) || !aligned(v, 8) || !aligned(C, 8) ||
                   (order && !aligned(order, 4))))
        return MPM_ERR_INVALID;
    // bounds line: every node total, and every product m v_d and m C_de, fits
    // int64 when np * max_mass * (max_speed + dim * max_affine * 3/2 + 1) < 2^62
    // (first-moment shares of one quantity sum to at most half of it in
    // magnitude, doubled by the middle share, plus one unit of rounding each)
    const long double line = (long double)np * (long double)max_mass *
                             ((long double)max_speed + (long double)dim * (long double)max_affine * 1.5L + 1.0L);
    const long double one = (long double)max_mass *
                            ((long double)max_speed + (long double)dim * (long double)max_affine * 1.5L + 1.0L);
    if (line >= 4611686018427387904.0L || one >= 4611686018427387904.0L)
        return MPM_ERR_OVERFLOW;
    return MPM_OK;
}

}  // namespace

extern "C" {

int mpm_p2g_isplit(int32_t dim, int32_t n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                   const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed, int64_t max_affine,
                   void *workspace, size_t workspace_bytes, int64_t *grid_out, uint32_t *status, hipStream_t stream)
{
    const int rc = check_isplit(dim, n, np, X, m, v, C, order, max_mass, max_speed, max_affine, grid_out, status);
    if (rc != MPM_OK)
        return rc;
    if (workspace) {
        if (!aligned(workspace, 256))
            return MPM_ERR_INVALID;
        if (workspace_bytes < isplit_layout(dim, n, np).total)
            return MPM_ERR_WORKSPACE;
        return hip_status(launch_p2g_isplit_tiled(dim, n, np, X, m, v, C, order, max_mass, max_speed, max_affine,
                                                  workspace, grid_out, status, stream));
    }
    return hip_status(launch_p2g_isplit(dim, n, np, X, m, v, C, order, max_mass, max_speed, max_affine, grid_out,
                                        status, stream));
}

int mpm_p2g_isplit_noalloc(int32_t dim, int32_t n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                           const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                           int64_t max_affine, int64_t *grid_out, uint32_t *status, hipStream_t stream)
{
    const int rc = check_isplit(dim, n, np, X, m, v, C, order, max_mass, max_speed, max_affine, grid_out, status);
    if (rc != MPM_OK)
        return rc;
    if (isplit_layout(dim, n, np).total > (size_t)MPM_ISPLIT_SCRATCH_BYTES)
        return MPM_ERR_SCRATCH;
    if (np == 0)
        return MPM_OK;
    void *ws = nullptr;
    const hipError_t e = isplit_scratch(&ws);
    if (e != hipSuccess)
        return MPM_ERR_HIP;
    return hip_status(launch_p2g_isplit_tiled(dim, n, np, X, m, v, C, order, max_mass, max_speed, max_affine, ws,
                                              grid_out, status, stream));
}

int mpm_grid_update(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, float *vg, float dt,
                    const float *gravity, int32_t sticky, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !aligned(grid_io, 8) || !aligned(vg, 4) || !gravity || sticky < 0 ||
        sticky > grid->n / 2 || (bins && !aligned(bins, 256)))
        return MPM_ERR_INVALID;
    float g3[3] = { gravity[0], gravity[1], grid->dim == 3 ? gravity[2] : 0.0f };
    if (!bins)
        return hip_status(launch_grid_update(grid->dim, grid->n, grid_io, vg, dt, g3, sticky, nullptr, stream));
    if (bins_bytes < fixed_prefix_bytes(grid))
        return MPM_ERR_WORKSPACE;
    mpm_ws_layout l;
    make_layout(grid, 0, &l);         // tile arrays and meta come first: their offsets do not depend on n
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    const BinView v = bin_view(bins, l, make_stamp(grid, 0, none, true));
    return hip_status(launch_grid_update(grid->dim, grid->n, grid_io, vg, dt, g3, sticky, &v, stream));
}

int mpm_grid_clear(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !aligned(grid_io, 8) || (bins && !aligned(bins, 256)))
        return MPM_ERR_INVALID;
    if (!bins)
        return hip_status(launch_grid_clear(grid->dim, grid->n, grid_io, nullptr, stream));
    if (bins_bytes < fixed_prefix_bytes(grid))
        return MPM_ERR_WORKSPACE;
    mpm_ws_layout l;
    make_layout(grid, 0, &l);         // tile arrays and meta come first: their offsets do not depend on n
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    const BinView v = bin_view(bins, l, make_stamp(grid, 0, none, true));
    return hip_status(launch_grid_clear(grid->dim, grid->n, grid_io, &v, stream));
}

int mpm_neohookean_affine(const mpm_grid_desc *grid, const mpm_particles *particles, const float *F, const float *vol0,
                          float dt, float mu, float lambda, float *C_out, uint32_t *status, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !particles || particles->n < 0 || particles->n > kMaxParticles)
        return MPM_ERR_INVALID;
    const int64_t np = particles->n;
    if (np > 0 && (!particles->C || !particles->m || !F || !vol0 || !C_out || !aligned(particles->C, 4) ||
                   !aligned(particles->m, 4) || !aligned(F, 4) || !aligned(vol0, 4) || !aligned(C_out, 4)))
        return MPM_ERR_INVALID;
    if (!aligned(status, 4) || !(dt >= 0.0f) || !(mu >= 0.0f) || !(lambda >= 0.0f))
        return MPM_ERR_INVALID;
    return hip_status(launch_neohookean_affine(grid->dim, grid->n, np, F, particles->C, particles->m, vol0, dt, mu,
                                               lambda, C_out, status, stream));
}

int mpm_update_deformation(const mpm_grid_desc *grid, const mpm_particles *particles, float *F, float dt,
                           hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !particles || particles->n < 0 || particles->n > kMaxParticles)
        return MPM_ERR_INVALID;
    if (particles->n > 0 && (!particles->C || !F || !aligned(particles->C, 4) || !aligned(F, 4)))
        return MPM_ERR_INVALID;
    return hip_status(launch_update_F(grid->dim, particles->n, particles->C, F, dt, stream));
}

int mpm_update_deformation_stress(const mpm_grid_desc *grid, const mpm_particles *particles, float *F,
                                  const float *vol0, float dt, float mu, float lambda, float *C_out, uint32_t *status,
                                  hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !particles || particles->n < 0 || particles->n > kMaxParticles)
        return MPM_ERR_INVALID;
    const int64_t np = particles->n;
    if (np > 0 && (!particles->C || !particles->m || !F || !vol0 || !C_out || !aligned(particles->C, 4) ||
                   !aligned(particles->m, 4) || !aligned(F, 4) || !aligned(vol0, 4) || !aligned(C_out, 4) ||
                   C_out == particles->C || C_out == F))
        return MPM_ERR_INVALID;
    if (!aligned(status, 4) || !(dt >= 0.0f) || !(mu >= 0.0f) || !(lambda >= 0.0f))
        return MPM_ERR_INVALID;
    return hip_status(launch_update_F_stress(grid->dim, grid->n, np, particles->C, F, particles->m, vol0, dt, mu,
                                             lambda, C_out, status, stream));
}

int mpm_g2p_update_deformation_stress(const mpm_grid_desc *grid, const float *vg, const mpm_particles *particles,
                                      float dt, float *F, const float *vol0, float mu, float lambda, float *C_out,
                                      uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, true)) != MPM_OK)
        return rc;
    const int64_t np = particles->n;
    if (!aligned(vg, 4) || !aligned(status, 4))
        return MPM_ERR_INVALID;
    if (np > 0 && (!particles->C || !F || !vol0 || !C_out || !aligned(particles->C, 4) || !aligned(F, 4) ||
                   !aligned(vol0, 4) || !aligned(C_out, 4) || C_out == particles->C || C_out == F))
        return MPM_ERR_INVALID;
    if (!(dt >= 0.0f) || !(mu >= 0.0f) || !(lambda >= 0.0f))
        return MPM_ERR_INVALID;
    return hip_status(launch_g2p_stress(grid->dim, grid->n, vg, particles->x, particles->v, particles->C, np, dt, F,
                                        particles->m, vol0, mu, lambda, C_out, status, stream));
}

int mpm_pbmpm_project_elastic(const mpm_grid_desc *grid, const mpm_particles *particles, const float *F, float relax,
                              int32_t polar_iters, uint32_t *status, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !particles || particles->n < 0 || particles->n > kMaxParticles)
        return MPM_ERR_INVALID;
    if (particles->n > 0 && (!aligned(particles->C, 4) || !aligned(F, 4)))
        return MPM_ERR_INVALID;
    if (!aligned(status, 4) || !(relax >= 0.0f && relax <= 2.0f) || polar_iters < 0 || polar_iters > 64)
        return MPM_ERR_INVALID;
    return hip_status(launch_pbmpm_project(grid->dim, particles->n, F, particles->C, relax, polar_iters, status,
                                           stream));
}

int mpm_pbmpm_g2p_project(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles, const float *F,
                          float relax, int32_t polar_iters, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, false)) != MPM_OK)
        return rc;
    if (!aligned(dg, 4) || !aligned(status, 4) || (particles->n > 0 && (!aligned(particles->C, 4) || !aligned(F, 4))))
        return MPM_ERR_INVALID;
    if (!(relax >= 0.0f && relax <= 2.0f) || polar_iters < 0 || polar_iters > 64)
        return MPM_ERR_INVALID;
    return hip_status(launch_pbmpm_g2p_project(grid->dim, grid->n, dg, particles->x, particles->v, particles->C,
                                               particles->n, F, relax, polar_iters, status, stream));
}

int mpm_pbmpm_g2p_project_records(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles,
                                  const float *F, float relax, int32_t polar_iters, const mpm_ranges *ranges, void *ws,
                                  size_t ws_bytes, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_ranges(ranges)) != MPM_OK ||
        (rc = check_particles(grid, particles, true, true)) != MPM_OK)
        return rc;
    if (!aligned(dg, 4) || !aligned(status, 4) || !aligned(ws, 256) ||
        (particles->n > 0 && (!aligned(particles->C, 4) || !aligned(F, 4))))
        return MPM_ERR_INVALID;
    if (!(relax >= 0.0f && relax <= 2.0f) || polar_iters < 0 || polar_iters > 64)
        return MPM_ERR_INVALID;
    if ((rc = mpm_check_bounds(grid, particles->n, ranges, nullptr)) != MPM_OK)
        return rc;
    mpm_ws_layout l;
    make_layout(grid, particles->n, &l);
    if (ws_bytes < l.total_bytes)
        return MPM_ERR_WORKSPACE;
    const RangesF rf = ranges_f(ranges);
    const BinView b = bin_view(ws, l, make_stamp(grid, particles->n, rf, false));
    return hip_status(launch_pbmpm_g2p_project(grid->dim, grid->n, dg, particles->x, particles->v, particles->C,
                                               particles->n, F, relax, polar_iters, status, stream, &b, rf,
                                               particles->m));
}

int mpm_pbmpm_grid_update(const mpm_grid_desc *grid, void *bins, size_t bins_bytes, int64_t *grid_io, float *dg,
                          int32_t band, hipStream_t stream)
{
    if (check_desc(grid) != MPM_OK || !aligned(grid_io, 8) || !aligned(dg, 4) || band < 1 ||
        2 * band >= grid->n - 1 || (bins && !aligned(bins, 256)))
        return MPM_ERR_INVALID;
    if (!bins)
        return hip_status(launch_pbmpm_grid_update(grid->dim, grid->n, grid_io, dg, band, nullptr, stream));
    if (bins_bytes < fixed_prefix_bytes(grid))
        return MPM_ERR_WORKSPACE;
    mpm_ws_layout l;
    make_layout(grid, 0, &l);
    const RangesF none{ 0.0f, 0.0f, 0.0f };
    const BinView v = bin_view(bins, l, make_stamp(grid, 0, none, true));
    return hip_status(launch_pbmpm_grid_update(grid->dim, grid->n, grid_io, dg, band, &v, stream));
}

int mpm_pbmpm_g2p_integrate(const mpm_grid_desc *grid, const float *dg, const mpm_particles *particles, float *F,
                            float dt, const float *gravity, uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, false)) != MPM_OK)
        return rc;
    if (!aligned(dg, 4) || !aligned(status, 4) || !gravity || !(dt >= 0.0f))
        return MPM_ERR_INVALID;
    if (particles->n > 0 && (!particles->C || !aligned(particles->C, 4) || !aligned(F, 4)))
        return MPM_ERR_INVALID;
    const float g3[3] = { gravity[0], gravity[1], grid->dim == 3 ? gravity[2] : 0.0f };
    return hip_status(launch_pbmpm_g2p_integrate(grid->dim, grid->n, dg, particles->x, particles->v, particles->C,
                                                 particles->n, F, dt, g3, status, stream));
}

int mpm_pbmpm_integrate(const mpm_grid_desc *grid, const mpm_particles *particles, float dt, const float *gravity,
                        uint32_t *status, hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, false)) != MPM_OK)
        return rc;
    if (!gravity || !aligned(status, 4) || !(dt >= 0.0f))
        return MPM_ERR_INVALID;
    const float g3[3] = { gravity[0], gravity[1], grid->dim == 3 ? gravity[2] : 0.0f };
    return hip_status(launch_pbmpm_integrate(grid->dim, grid->n, particles->n, particles->x, particles->v, dt, g3,
                                             status, stream));
}

int mpm_g2p(const mpm_grid_desc *grid, const float *vg, const mpm_particles *particles, float dt, uint32_t *status,
            hipStream_t stream)
{
    int rc;
    if ((rc = check_desc(grid)) != MPM_OK || (rc = check_particles(grid, particles, true, false)) != MPM_OK)
        return rc;
    if (!aligned(vg, 4) || !aligned(status, 4) || (particles->n > 0 && !particles->C))
        return MPM_ERR_INVALID;
    return hip_status(launch_g2p(grid->dim, grid->n, vg, particles->x, particles->v, particles->C, particles->n, dt,
                                 status, stream));
}

}  // extern "C"
