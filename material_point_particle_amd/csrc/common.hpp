// common.hpp -- device helpers and internal launch interfaces of libmpm.
//
// Everything here is gfx950 HIP.  The floating-point expressions below are
// the library's fixed operation order for the transfer; the build uses
// -ffp-contract=off and no fast-math, so each operation is one IEEE binary32
// (or binary64) operation rounded to nearest even, exactly as written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mpm.h"

namespace mpmk {

constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr int kWave = 64;
constexpr int kTile = 4;             // tile edge in cells
constexpr int kGroup = 4;            // records per group: one cell's particles, four at a time
constexpr int kRowSlots = kWave * kGroup;  // a row: one group per lane (256 group entries)
constexpr int kRowsPerItem = 8;      // most rows of one P2G work item (2048 group entries)
constexpr int kPlanTiles = 4096;     // tiles per block of binning's work-item plan
constexpr int kPlanStride = 2 + kRowsPerItem;  // words per plan block: records, full slices, slices per class

// One axis of a particle's quadratic B-spline stencil.  With g = x*n in node
// units, the stencil starts at base = floor(g - 1/2) ("Mass Matrix Assembly on
// Tensor Cores for Implicit PIC", shape functions: second-order support on
// {j-1, j, j+1} below a half-cell fraction, {j, j+1, j+2} above); f = g - base
// lies in [1/2, 3/2); the weights are the quadratic B-spline at distances f,
// f-1 and f-2, and r[o] = (o - f) dx is node base+o's offset from the particle.
struct Axis {
    float w0, w1, w2;
    float r0, r1, r2;
    int base;
};

__device__ __forceinline__ bool axis_stencil(float x, float nf, float dx, float last_base, Axis &s)
{
    const float g = x * nf;
    const float b = floorf(g - 0.5f);
    const bool ok = (b >= 0.0f) && (b <= last_base);
    const float f = g - b;
    const float t0 = 1.5f - f;
    const float t1 = f - 1.0f;
    const float t2 = f - 0.5f;
    s.w0 = 0.5f * (t0 * t0);
    s.w1 = 0.75f - (t1 * t1);
    s.w2 = 0.5f * (t2 * t2);
    s.r0 = (0.0f - f) * dx;
    s.r1 = (1.0f - f) * dx;
    s.r2 = (2.0f - f) * dx;
    s.base = ok ? (int)b : 0;
    return ok;
}

// Grid update of one node ("Implementation -- GPU Optimization & Reference
// Codebases", section 5 rules 1 and 7): where M != 0, v = (float)((double)P /
// (double)M) and then v + dt*g (gdt, formed once in float32); v = 0 where
// M == 0 and on the sticky walls.
__device__ __forceinline__ float node_velocity(int64_t M, int64_t P, float gdt, bool wall)
{
    float v = 0.0f;
    if (M != 0) {
        v = (float)((double)P / (double)M);
        v = v + gdt;
    }
    return wall ? 0.0f : v;
}

// APIC gather and advection of one particle (grid-to-particle).  Over the
// stencil in lexicographic node order (x offset outermost), with
// w = (wx[a]*wy[b])*wz[c] and wv_d = w*vel(a, b, c, d), the per-axis offset
// sums S[d][e][o] += wv_d; then v_d = sum_o S[d][0][o] and
// B_de = sum_o r_e[o] S[d][e][o] (in offset order), C = B*cscale,
// x_d + dt*v_d clamped to [lo, hi].  Returns whether a coordinate was clamped.
template <int DIM, class Vel>
__device__ __forceinline__ bool g2p_particle(const Axis (&ax)[DIM], const float (&x)[DIM], Vel &&vel, float dt,
                                             float lo, float hi, float cscale, float (&vn)[DIM],
                                             float (&Cn)[DIM * DIM], float (&xn)[DIM])
{
    // S[d][e][o]: sum of w * vg_d over the stencil nodes at offset o along
    // axis e, in lexicographic node order; v and B follow from it because
    // r_e depends on the offset along axis e only.
    float S[DIM][DIM][3];
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
#pragma unroll
            for (int o = 0; o < 3; ++o)
                S[d][e][o] = 0.0f;
    const float wx[3] = { ax[0].w0, ax[0].w1, ax[0].w2 }, rx[3] = { ax[0].r0, ax[0].r1, ax[0].r2 };
    const float wy[3] = { ax[1].w0, ax[1].w1, ax[1].w2 }, ry[3] = { ax[1].r0, ax[1].r1, ax[1].r2 };
    float wz[3] = { 1.0f, 0.0f, 0.0f }, rz[3] = { 0.0f, 0.0f, 0.0f };
    if constexpr (DIM == 3) {
        wz[0] = ax[2].w0; wz[1] = ax[2].w1; wz[2] = ax[2].w2;
        rz[0] = ax[2].r0; rz[1] = ax[2].r1; rz[2] = ax[2].r2;
    }
    const int nc = DIM == 3 ? 3 : 1;
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int c = 0; c < nc; ++c) {
                float w = wx[a] * wy[b];
                if constexpr (DIM == 3)
                    w = w * wz[c];
                const int o[3] = { a, b, c };
#pragma unroll
                for (int d = 0; d < DIM; ++d) {
                    const float wv = w * vel(a, b, c, d);
#pragma unroll
                    for (int e = 0; e < DIM; ++e)
                        S[d][e][o[e]] = S[d][e][o[e]] + wv;
                }
            }
    const float *rr[3] = { rx, ry, rz };
    bool clamped = false;
#pragma unroll
    for (int d = 0; d < DIM; ++d) {
        vn[d] = (S[d][0][0] + S[d][0][1]) + S[d][0][2];
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            Cn[d * DIM + e] = ((rr[e][0] * S[d][e][0] + rr[e][1] * S[d][e][1]) + rr[e][2] * S[d][e][2]) * cscale;
        const float xa = x[d] + dt * vn[d];
        xn[d] = fminf(fmaxf(xa, lo), hi);
        clamped = clamped || (xn[d] != xa);
    }
    return clamped;
}

// Declared ranges as float32 thresholds.  The host rounds each declared
// maximum down to the largest float not above it, so |value| <= threshold in
// float32 decides exactly what |value| <= maximum decides in real numbers.
// Floats per particle record of the binned copy: x, v, C, m padded to a
// multiple of four (64 bytes in 3D, 48 in 2D) so records load as float4s.
template <int DIM>
__host__ __device__ constexpr int rec_floats() { return ((2 * DIM + DIM * DIM + 1) + 3) / 4 * 4; }

// Local number of a cell inside its tile.  In 3D the cells are numbered x
// fastest, then z, then y: with the binned layout a dense tile puts cell l on
// lane ~l, and with this order the 64 lanes' node addresses in the 6x6x6 LDS
// block (x, y, z strides 1, 6, 36) fall in distinct LDS banks, so the
// stencil's LDS atomics run without bank conflicts (row-major order costs
// twice as long per instruction on gfx950).  2D tiles are row-major.
template <int DIM>
__host__ __device__ __forceinline__ uint32_t tile_local(const uint32_t l[DIM])
{
    if constexpr (DIM == 3)
        return l[0] + kTile * l[2] + kTile * kTile * l[1];
    else
        return l[0] + kTile * l[1];
}

template <int DIM>
__host__ __device__ __forceinline__ void tile_local_inverse(uint32_t local, uint32_t l[DIM])
{
    l[0] = local % kTile;
    if constexpr (DIM == 3) {
        l[2] = (local / kTile) % kTile;
        l[1] = local / (kTile * kTile);
    } else {
        l[1] = local / kTile;
    }
}

template <int DIM>
__host__ __device__ constexpr uint32_t cells_per_tile() { return DIM == 3 ? kTile * kTile * kTile : kTile * kTile; }

// Upper bound on the groups of kGroup same-cell entries formed from `count`
// records of one tile: each occupied cell adds at most kGroup-1 pad entries
// and at most min(count, cells) cells are occupied.  The bound depends on the
// count alone, so rows are laid out before the cells are sorted.
template <int DIM>
__host__ __device__ constexpr uint32_t groups_bound(uint32_t count)
{
    const uint64_t occupied = count < cells_per_tile<DIM>() ? count : cells_per_tile<DIM>();
    return (uint32_t)(((uint64_t)count + (kGroup - 1) * occupied) / kGroup);
}

template <int DIM>
__host__ __device__ inline uint32_t rows_bound(uint32_t count)
{
    return (groups_bound<DIM>(count) + kWave - 1) / kWave;
}

// Records per P2G work item: a tile's records are cut into slices of this
// many (the last one shorter); a full slice's groups fill exactly
// kRowsPerItem rows at the bound.
template <int DIM>
__host__ __device__ constexpr uint32_t slice_records()
{
    return kRowsPerItem * kRowSlots - (kGroup - 1) * cells_per_tile<DIM>();
}

struct RangesF {
    float max_mass, max_speed, max_affine;
};

// Inclusive prefix sum of v over the lanes of the wavefront.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += o;
    }
    return v;
}

// Count the lanes of the wavefront for which `pred` holds with one atomic.
__device__ __forceinline__ void wave_count(bool pred, uint32_t *counter)
{
    const unsigned long long bits = __ballot(pred);
    if (bits != 0ull && (threadIdx.x % kWave) == (unsigned)__ffsll((long long)bits) - 1u)
        atomicAdd(counter, (uint32_t)__popcll(bits));
}

// ---------------------------------------------------------------------------
// Internal launch interfaces (host side).  Arguments are validated by the
// C ABI layer before these are called; each returns hipGetLastError().
// ---------------------------------------------------------------------------
struct Fields {           // component-major particle arrays of n particles
    const float *x, *v, *C, *m;
    int64_t n;
};

// Words of the binning workspace's meta array (uint32[kMetaWords]).  It sits
// at an offset that does not depend on the particle count, so every entry
// point that is handed a workspace can find it.
constexpr int kMetaWords = 32;
constexpr int kMetaItems = 0;        // work items
constexpr int kMetaBinned = 2;       // binned particles
constexpr int kMetaCursor = 3;       // work cursor of P2G and the fused substep
constexpr int kMetaRuns = 6;         // runs (chunk, tile) the binning's count formed
constexpr int kMetaKeys = 7;         // 1: the binning wrote each record's cell key (cell_key)
// The binning writes the records' cell keys when the runs average at least
// this many records (input listed region by region, where the key bytes of a
// 128-byte line come from few runs); otherwise P2G reads each record's cell
// from its position.  Measured on the 16M-particle blob workload: the key
// bytes cost the scatter 56 us with runs of ~70 records (generator order) and
// 276 us with runs of ~11 (shuffled), reading cells from positions costs P2G
// ~80 us.
constexpr uint32_t kKeyRunLength = 32;
constexpr int kMetaStamp = 16;       // the binning's stamp (BinStamp)
constexpr uint32_t kStampMagic = 0x4D504D42u;

// What a binning was made for: written into meta by the binning, compared by
// every kernel that reads the bins before it reads anything else, so that a
// workspace binned for another grid, particle count or range declaration is
// refused on the device (status[3]) instead of being read with the wrong
// layout or bounds.  keep: records kept as they are (the resident binning),
// without range checks or the cell sort.
struct BinStamp {
    uint32_t magic, dim, n, np_lo, np_hi, max_mass, max_speed, max_affine, keep;
};
static_assert(sizeof(BinStamp) / 4 + kMetaStamp <= kMetaWords, "the stamp fits the meta words");

// ranges: also compare the declared ranges and require a checked binning
// (records range-checked), as the tiled P2G needs.
__device__ __forceinline__ bool stamp_matches(const uint32_t *meta, const BinStamp &s, bool ranges)
{
    const uint32_t *m = meta + kMetaStamp;
    bool ok = m[0] == s.magic && m[1] == s.dim && m[2] == s.n && m[3] == s.np_lo && m[4] == s.np_hi;
    if (ranges)
        ok = ok && m[5] == s.max_mass && m[6] == s.max_speed && m[7] == s.max_affine && m[8] == 0u;
    return ok;
}

struct BinView {          // the workspace arrays, as typed device pointers
    uint32_t *tile_count, *tile_start, *items, *meta, *rank, *slot, *scan_tmp;
    uint8_t *cell_key, *tile_active;
    float *sorted;
    int64_t n_cells, n_tiles, max_items, n_fields;
    BinStamp stamp;       // the binning this view is for (written by launch_bin, expected by readers)
};

hipError_t launch_p2g_direct(int dim, int n, int frac_bits, const Fields &p, const uint32_t *order, RangesF r,
                             int64_t *grid, uint32_t *status, hipStream_t s);
hipError_t launch_p2g_tiled(int dim, int n, int frac_bits, const BinView &b, int64_t *grid, uint32_t *status,
                            hipStream_t s);
hipError_t launch_g2p2g(int dim, int n, int frac_bits, const BinView &b, RangesF r, const int64_t *grid_in,
                        int64_t *grid_out, uint8_t *tiles_out, int64_t *grid_clear, uint8_t *tiles_clear, float dt,
                        const float *gravity, int sticky, uint32_t *status, hipStream_t s);
hipError_t launch_p2g_cic_split(int64_t n, const int32_t *X, const int32_t *m, const int32_t *vel,
                                const uint32_t *order, int cells, int64_t *grid, uint32_t *status, hipStream_t s);
hipError_t launch_p2g_isplit(int dim, int n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                             const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                             int64_t max_affine, int64_t *grid, uint32_t *status, hipStream_t s);
struct IsplitLayout {      // byte offsets into the integer-split workspace
    size_t count, start, partial, meta, rank, rec, total;
    int64_t tiles_x, tiles, entries, scan_blocks;
    int slot_shift;       // 2^slot_shift counters per tile
};
IsplitLayout isplit_layout(int dim, int n, int64_t np);
hipError_t isplit_scratch(void **ptr);
hipError_t launch_p2g_isplit_tiled(int dim, int n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                                   const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                                   int64_t max_affine, void *ws, int64_t *grid, uint32_t *status, hipStream_t s);
hipError_t launch_bin(int dim, int n, const Fields &p, RangesF r, const BinView &b, uint32_t *status,
                      hipStream_t s, bool keep = false);
hipError_t launch_gather_records(int dim, int64_t np, const BinView &b, float *x, float *v, float *C,
                                 uint32_t *status, hipStream_t s);
hipError_t launch_grid_update(int dim, int n, int64_t *grid, float *vg, float dt, const float *gravity,
                              int sticky, const BinView *bins, hipStream_t s);
hipError_t launch_grid_clear(int dim, int n, int64_t *grid, const BinView *bins, hipStream_t s);
hipError_t launch_grid_clear_tiles(int dim, int n, int64_t *grid, uint8_t *tiles, hipStream_t s);
hipError_t launch_neohookean_affine(int dim, int n, int64_t np, const float *F, const float *C, const float *m,
                                    const float *vol0, float dt, float mu, float lambda, float *Cout,
                                    uint32_t *status, hipStream_t s);
hipError_t launch_update_F(int dim, int64_t np, const float *C, float *F, float dt, hipStream_t s);
hipError_t launch_g2p(int dim, int n, const float *vg, float *x, float *v, float *C, int64_t np, float dt,
                      uint32_t *status, hipStream_t s);
hipError_t launch_pbmpm_project(int dim, int64_t np, const float *F, float *D, float relax, int polar_iters,
                                uint32_t *status, hipStream_t s);
hipError_t launch_pbmpm_grid_update(int dim, int n, int64_t *grid, float *dg, int band, const BinView *bins,
                                    hipStream_t s);
hipError_t launch_pbmpm_integrate(int dim, int n, int64_t np, float *x, float *d, float dt, const float *gravity,
                                  uint32_t *status, hipStream_t s);

int device_cu_count();

}  // namespace mpmk
