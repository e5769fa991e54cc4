// fused.hip -- the fused grid-to-particle / particle-to-grid substep kernel
// over the resident binned records.
#include "p2g_device.hpp"

namespace mpmk {
namespace {

// ---------------------------------------------------------------------------
// Fused grid-to-particle and particle-to-grid per work item ("Implementation
// -- GPU Optimization & Reference Codebases", section 2.1: one kernel per
// tile slice loads the tile's node block with its halo, applying the grid
// update as it loads, gathers and updates the slice's particles, and scatters
// them into the next grid through the on-chip block).  The particle state is
// the binned records, updated in place.  Per item:
//  1. the grid velocity of the (kTile+4)^dim nodes t0-1 .. t0+6 per axis,
//     t0 the tile's first node (every node a particle of the tile reads
//     while it stays within a cell of the tile), is formed from grid_in with
//     node_velocity into LDS (sharing the node block's memory);
//  2. each record is gathered and advected (g2p_particle, the same arithmetic
//     as the G2P kernel; a particle whose stencil leaves that window reads
//     grid_in directly) and written back; its cell in the new position is its
//     key, or a stray mark when it has left the tile;
//  3. the keys are sorted on chip as in the P2G kernel and the rows deposit
//     the updated records into the tile's node block (range checks here, not
//     at binning); strays deposit with global atomics;
//  4. the block is flushed to grid_out, and every node tile this item wrote
//     is flagged in tiles_out (for the restricted clear of that grid later);
//  5. (after the last item, with a third grid) the flagged node tiles of the
//     grid read in the previous substep are zeroed, so that three grids in
//     turn need no clear between substeps.
// With grid_in NULL only steps 2 (keys), 3 and 4 run: the deposit of the
// records as they are.
// ---------------------------------------------------------------------------
struct FusedArgs {
    TiledArgs t;               // sorted: the records; grid: grid_out
    float *records;            // the same records, written
    const int64_t *grid_in;    // grid velocity source, or NULL for a deposit only
    uint8_t *tiles_out;        // node-tile flags of grid_out
    int64_t *grid_clear;       // a third grid to zero (its flagged node tiles), or NULL
    uint8_t *tiles_clear;      // its node-tile flags, reset with it
    RangesF r;
    float dt, lo, hi, cscale;
    float gdt[3];
    int sticky;
};

// Flags the node tiles covering nodes [lo, lo + span) per axis.
template <int DIM>
__device__ __forceinline__ void flag_node_tiles(uint8_t *tiles, int ntx, const int (&lo)[3], int span)
{
    int t0[3] = { 0, 0, 0 }, t1[3] = { 0, 0, 0 };
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        t0[e] = lo[e] / kTile;
        t1[e] = (lo[e] + span - 1) / kTile;
        t1[e] = t1[e] < ntx - 1 ? t1[e] : ntx - 1;
    }
    for (int z = t0[2]; z <= (DIM == 3 ? t1[2] : 0); ++z)
        for (int y = t0[1]; y <= t1[1]; ++y)
            for (int x = t0[0]; x <= t1[0]; ++x)
                tiles[((int64_t)z * ntx + y) * ntx + x] = 1;
}

template <int DIM>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
g2p2g_kernel(FusedArgs f)
{
    using TS = TileShape<DIM>;
    constexpr int R = rec_floats<DIM>();
    constexpr int W = kTile + 4;                                     // velocity window edge
    constexpr int WN = DIM == 3 ? W * W * W : W * W;
    constexpr int kFlush = (TS::nodes + kWave - 1) / kWave;
    static_assert(DIM * WN * sizeof(float) <= TS::ch * TS::nodes * sizeof(double),
                  "the velocity window fits in the node block's memory");
    __shared__ double acc[TS::ch * TS::nodes];                      // velocity window, then the node block
    __shared__ __align__(16) uint16_t ent[kMaxGroups * kGroup + 4];
    __shared__ uint16_t gpos[kMaxGroups];
    __shared__ uint32_t cnt[2 * kWave], cgs[kWave], rep[2 * kWave];
    __shared__ __align__(4) uint8_t keys[kKeyWords * kWave * 4];
    __shared__ uint16_t strays[slice_records<DIM>()];
    __shared__ uint32_t n_strays;
    static_assert(slice_records<DIM>() <= kKeyWords * kWave * 4, "a slice's keys fit the key buffer");
    const TiledArgs &a = f.t;
    float *vw = reinterpret_cast<float *>(acc);
    const int lane = threadIdx.x;
    // a workspace binned for another grid or particle count: refused before
    // anything else is read (the whole call does nothing)
    if (!stamp_matches(a.meta, a.stamp, false)) {
        if (blockIdx.x == 0 && lane == 0)
            atomicAdd(&a.status[3], 1u);
        return;
    }
    const uint32_t n_items = a.meta[kMetaItems];
    const int n = a.n;
    const int64_t nodes = DIM == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    for (int i = lane; i < TS::ch * TS::nodes; i += kWave)
        acc[i] = 0.0;
    cnt[lane] = 0u;
    cnt[kWave + lane] = 0u;
    __syncthreads();
    const uint4 *items = reinterpret_cast<const uint4 *>(a.items);
    for (;;) {
        uint32_t next = 0;
        if (lane == 0)
            next = atomicAdd(a.cursor, 1u);
        const uint32_t item = __builtin_amdgcn_readfirstlane(next);
        if (item >= n_items)
            break;
        const uint4 it = items[item];
        const uint32_t tile = it.x, first = it.y, count = it.z;
        int torg[3] = { 0, 0, 0 };
        {
            uint32_t t = tile;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                torg[e] = (int)(t % (uint32_t)a.ntx) * kTile;
                t /= (uint32_t)a.ntx;
            }
        }
        // 1. grid velocity of the window (its origin one node below the tile):
        //    every lane's nodes are loaded before any is converted, so the
        //    loads are in flight together
        if (f.grid_in) {
            constexpr int kWin = (WN + kWave - 1) / kWave;            // window nodes per lane
            int64_t M[kWin], P[kWin][DIM];
            bool wall[kWin];
#pragma unroll
            for (int m = 0; m < kWin; ++m) {
                const int i = lane + kWave * m;
                const int l[3] = { i % W, (i / W) % W, DIM == 3 ? i / (W * W) : 0 };
                bool inside = i < WN;
                wall[m] = false;
                int g[3] = { 0, 0, 0 };
#pragma unroll
                for (int e = 0; e < DIM; ++e) {
                    g[e] = torg[e] - 1 + l[e];
                    inside = inside && g[e] >= 0 && g[e] < n;
                    wall[m] = wall[m] || g[e] < f.sticky || g[e] >= n - f.sticky;
                }
                const int64_t node = DIM == 3 ? ((int64_t)g[2] * n + g[1]) * n + g[0] : (int64_t)g[1] * n + g[0];
                M[m] = inside ? f.grid_in[node] : 0;
#pragma unroll
                for (int d = 0; d < DIM; ++d)
                    P[m][d] = inside ? f.grid_in[(1 + d) * nodes + node] : 0;
            }
#pragma unroll
            for (int m = 0; m < kWin; ++m) {
                const int i = lane + kWave * m;
                if (i < WN) {
#pragma unroll
                    for (int d = 0; d < DIM; ++d)
                        vw[d * WN + i] = node_velocity(M[m], P[m][d], f.gdt[d], wall[m]);
                }
            }
        }
        if (lane == 0)
            n_strays = 0u;
        __syncthreads();
        // 2. gather and advect each record (with grid_in), then its key
        uint32_t clamps = 0;
        for (uint32_t i = (uint32_t)lane; i < count; i += kWave) {
            float4 *src = reinterpret_cast<float4 *>(f.records + (int64_t)(first + i) * R);
            float rec[R];
#pragma unroll
            for (int q = 0; q < R / 4; ++q) {
                const float4 t = src[q];
                rec[4 * q] = t.x;
                rec[4 * q + 1] = t.y;
                rec[4 * q + 2] = t.z;
                rec[4 * q + 3] = t.w;
            }
            if (f.grid_in) {
                Axis ax[DIM];
                float xp[DIM];
                bool win = true;
                int lb[3] = { 0, 0, 0 };
#pragma unroll
                for (int e = 0; e < DIM; ++e) {
                    xp[e] = rec[e];
                    axis_stencil(xp[e], a.nf, a.dx, a.last_base, ax[e]);
                    lb[e] = ax[e].base - (torg[e] - 1);
                    win = win && lb[e] >= 0 && lb[e] <= W - 3;
                }
                auto vel = [&](int aa, int b, int c, int d) {
                    if (win) {
                        const int w = DIM == 3 ? ((lb[2] + c) * W + (lb[1] + b)) * W + (lb[0] + aa)
                                               : (lb[1] + b) * W + (lb[0] + aa);
                        return vw[d * WN + w];
                    }
                    const int g[3] = { ax[0].base + aa, ax[1].base + b, DIM == 3 ? ax[DIM - 1].base + c : 0 };
                    const int64_t node = DIM == 3 ? ((int64_t)g[2] * n + g[1]) * n + g[0] : (int64_t)g[1] * n + g[0];
                    bool wall = false;
#pragma unroll
                    for (int e = 0; e < DIM; ++e)
                        wall = wall || g[e] < f.sticky || g[e] >= n - f.sticky;
                    const int64_t M = f.grid_in[node];
                    const int64_t P = M != 0 ? f.grid_in[(1 + d) * nodes + node] : 0;
                    return node_velocity(M, P, f.gdt[d], wall);
                };
                float vn[DIM], Cn[DIM * DIM], xn[DIM];
                clamps += g2p_particle<DIM>(ax, xp, vel, f.dt, f.lo, f.hi, f.cscale, vn, Cn, xn) ? 1u : 0u;
#pragma unroll
                for (int d = 0; d < DIM; ++d) {
                    rec[d] = xn[d];
                    rec[DIM + d] = vn[d];
                }
#pragma unroll
                for (int q = 0; q < DIM * DIM; ++q)
                    rec[2 * DIM + q] = Cn[q];
#pragma unroll
                for (int q = 0; q < R / 4; ++q)
                    src[q] = make_float4(rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3]);
            }
            uint32_t l[DIM];
            bool in_tile = true;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                Axis ax;
                axis_stencil(rec[e], a.nf, a.dx, a.last_base, ax);
                const int d = ax.base - torg[e];
                in_tile = in_tile && d >= 0 && d < kTile;
                l[e] = (uint32_t)(d & (kTile - 1));
            }
            keys[i] = in_tile ? (uint8_t)tile_local<DIM>(l) : (uint8_t)0xFFu;
            if (!in_tile)
                strays[atomicAdd(&n_strays, 1u)] = (uint16_t)i;
        }
        if (clamps != 0u)
            atomicAdd(&a.status[2], clamps);
        // the records written above are read back below by other lanes of
        // this workgroup: the barrier's workgroup-scope fence orders them
        __syncthreads();
        if (f.grid_in) {                                             // the window becomes the node block
            for (int i = lane; i < TS::ch * TS::nodes; i += kWave)
                acc[i] = 0.0;
            __syncthreads();
        }
        // 3. sort by the new cells and deposit
        uint32_t kw[kKeyWords];
        {
            const uint32_t *kwords = reinterpret_cast<const uint32_t *>(keys);
            const uint32_t n_words = (count + 3u) / 4u;
#pragma unroll
            for (int k = 0; k < kKeyWords; ++k) {
                const uint32_t i = (uint32_t)(k * kWave + lane);
                kw[k] = i < n_words ? kwords[i] : 0u;
            }
        }
        const uint32_t groups = sort_item<true>(kw, 0u, count, ent, gpos, cnt, cgs, rep, lane);
        const uint32_t rows = (groups + kWave - 1) / kWave;
        item_rows<DIM, true>(a, f.r, first, rows, groups, ent, acc, torg, lane);
        const uint32_t ns = n_strays;
        uint32_t bad = 0;
        for (uint32_t k = (uint32_t)lane; k < ns; k += kWave) {
            const float *rec = a.sorted + (int64_t)(first + strays[k]) * R;
            Particle<DIM> p;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                p.x[e] = rec[e];
                p.v[e] = rec[DIM + e];
            }
#pragma unroll
            for (int q = 0; q < DIM * DIM; ++q)
                p.C[q] = rec[2 * DIM + q];
            p.m = rec[2 * DIM + DIM * DIM];
            if (!in_ranges<DIM>(p, f.r)) {
                ++bad;
                continue;
            }
            Hoisted<DIM> h;
            hoist<DIM>(p, a.nf, a.dx, a.last_base, a.S, h);
            deposit_direct<DIM>(h, n, nodes, a.grid);
            const int lo[3] = { h.base[0], h.base[1], DIM == 3 ? h.base[DIM - 1] : 0 };
            flag_node_tiles<DIM>(f.tiles_out, a.ntx, lo, 3);
        }
        if (bad != 0u)
            atomicAdd(&a.status[1], bad);
        __syncthreads();
        // 4. flush the node block; flag its node tiles
#pragma unroll
        for (int m = 0; m < kFlush; ++m) {
            const int i = lane + kWave * m;
            if (i >= TS::nodes)
                continue;
            const int gx = torg[0] + i % TS::side, gy = torg[1] + (i / TS::side) % TS::side;
            const int gz = torg[2] + (DIM == 3 ? i / (TS::side * TS::side) : 0);
            const bool in_grid = gx < n && gy < n && gz < n;
            const int64_t node = DIM == 3 ? ((int64_t)gz * n + gy) * n + gx : (int64_t)gy * n + gx;
#pragma unroll
            for (int ch = 0; ch < TS::ch; ++ch) {
                const double val = acc[ch * TS::nodes + i];
                acc[ch * TS::nodes + i] = 0.0;
                if (val != 0.0 && in_grid)
                    atomic_add_i64(&a.grid[ch * nodes + node], (int64_t)val);
            }
        }
        if (lane == 0)
            flag_node_tiles<DIM>(f.tiles_out, a.ntx, torg, TS::side);
        __syncthreads();
    }
    // 5. With a third grid (the one read in the previous substep): once the
    //    item queue is empty, each workgroup zeroes the flagged node tiles of
    //    its share of that grid's tiles and resets their flags, so that no
    //    clear runs between substeps and the workgroups that finish first
    //    fill the kernel's tail with it.  This kernel neither reads nor
    //    writes that grid otherwise.
    if (f.grid_clear) {
        constexpr int kTileNodes = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
        static_assert(kTileNodes <= kWave, "one lane per node of a node tile");
        const int ntx = a.ntx;
        const int64_t n_tiles = DIM == 3 ? (int64_t)ntx * ntx * ntx : (int64_t)ntx * ntx;
        const int64_t share = (n_tiles + gridDim.x - 1) / gridDim.x;
        const int64_t t_begin = (int64_t)blockIdx.x * share;
        const int64_t t_end = t_begin + share < n_tiles ? t_begin + share : n_tiles;
        const int lx = lane % kTile, ly = (lane / kTile) % kTile, lz = DIM == 3 ? lane / (kTile * kTile) : 0;
        for (int64_t base = t_begin; base < t_end; base += kWave) {
            const int64_t t = base + lane;
            const bool flagged = t < t_end && f.tiles_clear[t] != 0;
            uint64_t m = __ballot(flagged);
            while (m != 0ull) {
                int64_t tt = base + __builtin_ctzll(m);
                m &= m - 1ull;
                const int tx = (int)(tt % ntx);
                tt /= ntx;
                const int ty = (int)(tt % ntx), tz = DIM == 3 ? (int)(tt / ntx) : 0;
                if (lane < kTileNodes) {
                    const int gx = tx * kTile + lx, gy = ty * kTile + ly, gz = tz * kTile + lz;
                    const int64_t node = DIM == 3 ? ((int64_t)gz * n + gy) * n + gx : (int64_t)gy * n + gx;
#pragma unroll
                    for (int ch = 0; ch < TS::ch; ++ch)
                        f.grid_clear[ch * nodes + node] = 0;
                }
            }
            if (flagged)
                f.tiles_clear[t] = 0;
        }
    }
}

}  // namespace

hipError_t launch_g2p2g(int dim, int n, int frac_bits, const BinView &b, RangesF r, const int64_t *grid_in,
                        int64_t *grid_out, uint8_t *tiles_out, int64_t *grid_clear, uint8_t *tiles_clear, float dt,
                        const float *gravity, int sticky, uint32_t *status, hipStream_t s)
{
    FusedArgs f;
    TiledArgs &a = f.t;
    a.sorted = b.sorted;
    a.cell_key = b.cell_key;
    a.items = b.items;
    a.meta = b.meta;
    a.stamp = b.stamp;
    a.cursor = b.meta + kMetaCursor;
    a.n = n;
    a.ntx = n / kTile;
    a.nf = (float)n;
    a.dx = 1.0f / (float)n;
    a.last_base = (float)(n - 3);
    a.S = ldexpf(1.0f, frac_bits);
    a.grid = grid_out;
    a.status = status;
    f.records = b.sorted;
    f.grid_in = grid_in;
    f.tiles_out = tiles_out;
    f.grid_clear = grid_clear;
    f.tiles_clear = tiles_clear;
    f.r = r;
    f.dt = dt;
    f.lo = a.dx;
    f.hi = (float)(n - 2) * a.dx;
    f.cscale = 4.0f * (float)n * (float)n;
    for (int d = 0; d < 3; ++d)
        f.gdt[d] = d < dim ? dt * gravity[d] : 0.0f;
    f.sticky = sticky;
    hipLaunchKernelGGL(reset_cursor_kernel, dim3(1), dim3(1), 0, s, a.cursor);
    int per_cu = 0;
    hipError_t e;
    if (dim == 3)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g2p2g_kernel<3>, kWave, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g2p2g_kernel<2>, kWave, 0);
    if (e != hipSuccess)
        return e;
    int64_t blocks = (int64_t)device_cu_count() * (per_cu > 0 ? per_cu : 1);
    if (blocks > b.max_items)
        blocks = b.max_items;
    if (blocks < 1)
        blocks = 1;
    if (dim == 3)
        hipLaunchKernelGGL(g2p2g_kernel<3>, dim3((unsigned)blocks), dim3(kWave), 0, s, f);
    else
        hipLaunchKernelGGL(g2p2g_kernel<2>, dim3((unsigned)blocks), dim3(kWave), 0, s, f);
    return hipGetLastError();
}

}  // namespace mpmk
