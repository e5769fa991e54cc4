// p2g.hip -- particle-to-grid scatter kernels for gfx950: the direct and
// tiled P2G paths (their shared device code and the transfer's fixed
// operation order are in p2g_device.hpp) and the integer-split
// cloud-in-cell scatter.
#include "p2g_device.hpp"

namespace mpmk {
namespace {

// ---------------------------------------------------------------------------
// Tiled path: one wavefront per work item (a slice of one tile's records),
// items taken from a work cursor.  Per item: the slice's records sorted by
// cell on chip into groups of four same-cell records (sort_item; a cell's last
// group completed with pad entries read with zero mass: records are
// range-checked at binning, so a pad's velocity and affine entries are finite
// and its products exact zeros); per row and lane, the group's contributions
// per stencil node and channel rounded and summed exactly in float64
// registers, one LDS atomic per node and channel into the tile's node block;
// then the block flushed with one 64-bit global atomic per non-zero node and
// channel and left zeroed.
template <int DIM>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
p2g_tiled_kernel(TiledArgs a)
{
    using TS = TileShape<DIM>;
    constexpr int R = rec_floats<DIM>();
    constexpr int G = kGroup;
    constexpr int kFlush = (TS::nodes + kWave - 1) / kWave;      // node-block entries per lane
    __shared__ double acc[TS::ch * TS::nodes];
    __shared__ __align__(16) uint16_t ent[kMaxGroups * kGroup + 4];
    __shared__ uint16_t gpos[kMaxGroups];
    __shared__ uint32_t cnt[2 * kWave], cgs[kWave], rep[2 * kWave];   // [kWave, 2 kWave): spare slots
    static_assert(slice_records<DIM>() < kPad16, "a slice offset must leave the pad bit free");
    static_assert((slice_records<DIM>() + 6) / 4 <= (uint32_t)(kWave * kKeyWords), "a slice's keys fit the key words");
    static_assert(groups_bound<DIM>(slice_records<DIM>()) <= kMaxGroups, "a slice's groups fit the entry rows");
    static_assert(cells_per_tile<DIM>() <= (uint32_t)kWave, "one lane per cell of a tile");
    const int lane = threadIdx.x;
    // bins made for another grid, particle count or range declaration, or by
    // the resident binning: refused before anything else is read
    if (!stamp_matches(a.meta, a.stamp, true)) {
        if (blockIdx.x == 0 && lane == 0)
            atomicAdd(&a.status[3], 1u);
        return;
    }
    const uint32_t n_items = a.meta[kMetaItems];
    const int64_t nodes = DIM == 3 ? (int64_t)a.n * a.n * a.n : (int64_t)a.n * a.n;

    // The block's local coordinates of the nodes this lane flushes (node
    // lane + 64*m of the block), fixed for every item.
    int fx[kFlush], fy[kFlush], fz[kFlush];
#pragma unroll
    for (int m = 0; m < kFlush; ++m) {
        const int i = lane + kWave * m;
        fx[m] = i % TS::side;
        fy[m] = (i / TS::side) % TS::side;
        fz[m] = DIM == 3 ? i / (TS::side * TS::side) : 0;
    }
    for (int i = lane; i < TS::ch * TS::nodes; i += kWave)
        acc[i] = 0.0;
    cnt[lane] = 0u;
    cnt[kWave + lane] = 0u;
    __syncthreads();

    // Lane 0 fetches the next item index as soon as an item starts; the next
    // item's record is loaded during the current item's rows and its cell keys
    // (from its records' positions) during the current item's flush, so no
    // round trip stalls the wave between items.
    const uint4 *items = reinterpret_cast<const uint4 *>(a.items);
    auto tile_origin = [&](uint32_t tile, int (&torg)[3]) {
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            torg[e] = (int)(tile % (uint32_t)a.ntx) * kTile;
            tile /= (uint32_t)a.ntx;
        }
    };
    uint32_t next = 0;
    if (lane == 0)
        next = atomicAdd(a.cursor, 1u);
    uint32_t item = __builtin_amdgcn_readfirstlane(next);
    // cell keys: from the binning's key array where it wrote one, else from
    // the records' positions
    const bool key_array = a.meta[kMetaKeys] != 0u;
    auto item_keys = [&](const uint4 &it, uint32_t (&kw)[kKeyWords]) {
        if (key_array) {
            load_keys(a.cell_key, it.y, it.z, lane, kw);
        } else {
            int t0[3] = { 0, 0, 0 };
            tile_origin(it.x, t0);
            record_keys<DIM>(a.sorted, it.y, it.z, t0, a.nf, lane, kw);
        }
    };
    uint4 rec_item = make_uint4(0u, 0u, 0u, 0u);
    uint32_t kw[kKeyWords];
    if (item < n_items) {
        rec_item = items[item];
        item_keys(rec_item, kw);
    }
    for (;;) {
        if (item >= n_items)
            break;
        if (lane == 0)
            next = atomicAdd(a.cursor, 1u);
        // item: tile, first record, records (one slice of the tile)
        const uint32_t first = rec_item.y, count = rec_item.z;
        int torg[3] = { 0, 0, 0 };
        tile_origin(rec_item.x, torg);
        const uint32_t groups = sort_item<false>(kw, first, count, ent, gpos, cnt, cgs, rep, lane);
        const uint32_t rows = (groups + kWave - 1) / kWave;
        const uint32_t item_next = __builtin_amdgcn_readfirstlane(next);
        uint4 rec_next = make_uint4(0u, 0u, 0u, 0u);
        if (item_next < n_items)
            rec_next = items[item_next];
        // The rows: the same loop as item_rows<DIM, false> in p2g_device.hpp,
        // kept here because that function, inlined into this kernel, was
        // scheduled differently and measured 12% slower on the blob workload.
        static_assert(kGroup == 4, "a group's entries load as one 8-byte word");
        for (uint32_t j = 0; j < rows; ++j) {
            // this lane's group in row j is group 64 j + lane of the item
            if (j * kWave + (uint32_t)lane >= groups)
                continue;
            const uint2 w2 = *reinterpret_cast<const uint2 *>(&ent[(j * kWave + lane) * kGroup]);
            const uint32_t e4[G] = { w2.x & 0xFFFFu, w2.x >> 16, w2.y & 0xFFFFu, w2.y >> 16 };
            GroupHoist<DIM> h[G];
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const float4 *src =
                    reinterpret_cast<const float4 *>(a.sorted + (int64_t)(first + (e4[k] & ~(uint32_t)kPad16)) * R);
                float rec[R];
#pragma unroll
                for (int q = 0; q < R / 4; ++q) {
                    const float4 t = src[q];
                    rec[4 * q] = t.x;
                    rec[4 * q + 1] = t.y;
                    rec[4 * q + 2] = t.z;
                    rec[4 * q + 3] = t.w;
                }
                if (e4[k] & kPad16)                          // completes the cell's group: zero mass
                    rec[2 * DIM + DIM * DIM] = 0.0f;
                group_hoist<DIM>(rec, a.nf, a.dx, a.last_base, a.S, h[k]);
            }
            // every record of the group is in one cell of this tile (binning's
            // invariant); a group that breaks it is counted and skipped
            bool ok = true;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                ok = ok && (unsigned)(h[0].base[e] - torg[e]) < (unsigned)kTile;
#pragma unroll
                for (int k = 1; k < G; ++k)
                    ok = ok && h[k].base[e] == h[0].base[e];
            }
            if (!ok) {
                atomicAdd(&a.status[3], 1u);
                continue;
            }
            int lb;
            if constexpr (DIM == 3)
                lb = ((h[0].base[2] - torg[2]) * TS::side + (h[0].base[1] - torg[1])) * TS::side +
                     (h[0].base[0] - torg[0]);
            else
                lb = (h[0].base[1] - torg[1]) * TS::side + (h[0].base[0] - torg[0]);
            const int nc = DIM == 3 ? 3 : 1;
#pragma unroll
            for (int aa = 0; aa < 3; ++aa)
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    float mwxy[G], t2[G][DIM];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        mwxy[k] = h[k].mwx[aa] * h[k].wy[b];
#pragma unroll
                        for (int d = 0; d < DIM; ++d)
                            t2[k][d] = h[k].t1[d][aa] + h[k].cy[d][b];
                    }
#pragma unroll
                    for (int c = 0; c < nc; ++c) {
                        const int off = DIM == 3 ? (c * TS::side + b) * TS::side + aa : b * TS::side + aa;
                        // The node's (1+DIM) x G contributions are independent until
                        // the per-channel sums; they are written phase by phase
                        // (products, rounding, widening, sums) so that the chains
                        // interleave instead of running back to back.
                        float wmS[G], val[1 + DIM][G];
#pragma unroll
                        for (int k = 0; k < G; ++k) {
                            wmS[k] = DIM == 3 ? mwxy[k] * h[k].wz[c] : mwxy[k];
                            val[0][k] = wmS[k];
                        }
#pragma unroll
                        for (int d = 0; d < DIM; ++d)
#pragma unroll
                            for (int k = 0; k < G; ++k) {
                                const float u = DIM == 3 ? t2[k][d] + h[k].cz[d][c] : t2[k][d];
                                val[1 + d][k] = wmS[k] * u;
                            }
                        double q[1 + DIM][G];
#pragma unroll
                        for (int ch = 0; ch < 1 + DIM; ++ch)
#pragma unroll
                            for (int k = 0; k < G; ++k)
                                q[ch][k] = (double)rintf(val[ch][k]);
#pragma unroll
                        for (int ch = 0; ch < 1 + DIM; ++ch) {
                            // exact integer adds: a pairwise tree gives the same sum
                            const double sum = (q[ch][0] + q[ch][1]) + (q[ch][2] + q[ch][3]);
                            atomicAdd(&acc[ch * TS::nodes + lb + off], sum);
                        }
                    }
                }
        }
        __syncthreads();
        item = item_next;
        rec_item = rec_next;
        if (item < n_items)
            item_keys(rec_item, kw);
        // Flush: every non-zero node sum goes to the grid with one 64-bit
        // atomic, and the block is left zeroed for the next item.
#pragma unroll
        for (int m = 0; m < kFlush; ++m) {
            const int i = lane + kWave * m;
            if (i >= TS::nodes)
                continue;
            const int gx = torg[0] + fx[m], gy = torg[1] + fy[m], gz = torg[2] + fz[m];
            const bool in_grid = gx < a.n && gy < a.n && gz < a.n;
            const int64_t node = DIM == 3 ? ((int64_t)gz * a.n + gy) * a.n + gx : (int64_t)gy * a.n + gx;
#pragma unroll
            for (int ch = 0; ch < TS::ch; ++ch) {
                const double val = acc[ch * TS::nodes + i];
                acc[ch * TS::nodes + i] = 0.0;
                if (val != 0.0 && in_grid)
                    atomic_add_i64(&a.grid[ch * nodes + node], (int64_t)val);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Integer-split cloud-in-cell ("particle to grid transfer in checked integer
// arithmetic"): for q in {m, m*vx, m*vy}, far = round(q*fx / 2^16) with ties
// to even, near = q - far; each part is split along y the same way.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t round_shift16_even(int64_t t)
{
    const int64_t fl = t >> 16;            // floor(t / 65536): arithmetic shift
    const int64_t r = t & 0xFFFF;          // t - 65536*fl, in [0, 65536)
    return fl + ((r > 0x8000) | ((r == 0x8000) & (fl & 1)));
}

__global__ void __launch_bounds__(256) p2g_cic_split_kernel(int64_t n, const int32_t *__restrict__ X,
                                                             const int32_t *__restrict__ m,
                                                             const int32_t *__restrict__ vel,
                                                             const uint32_t *__restrict__ order, int cells,
                                                             int64_t *__restrict__ grid, uint32_t *__restrict__ status)
{
    const int64_t nn = cells + 1;
    const int64_t span = (int64_t)cells << 16;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = order ? (int64_t)order[k] : k;
        if (p >= n) {                    // an order entry that names no particle
            atomicAdd(&status[3], 1u);
            continue;
        }
        const int64_t px = X[p], py = X[n + p];
        const bool ok = px >= 0 && px < span && py >= 0 && py < span;
        wave_count(!ok, &status[0]);
        if (!ok)
            continue;
        const int64_t cx = px >> 16, cy = py >> 16;
        const int64_t fx = px & 0xFFFF, fy = py & 0xFFFF;
        const int64_t q[3] = { (int64_t)m[p], (int64_t)m[p] * vel[p], (int64_t)m[p] * vel[n + p] };
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const int64_t qx1 = round_shift16_even(q[c] * fx);
            const int64_t qx0 = q[c] - qx1;
            const int64_t q01 = round_shift16_even(qx0 * fy);
            const int64_t q11 = round_shift16_even(qx1 * fy);
            int64_t *g = grid + c * nn * nn;
            atomic_add_i64(&g[cy * nn + cx], qx0 - q01);
            atomic_add_i64(&g[(cy + 1) * nn + cx], q01);
            atomic_add_i64(&g[cy * nn + cx + 1], qx1 - q11);
            atomic_add_i64(&g[(cy + 1) * nn + cx + 1], q11);
        }
    }
}

int grid_blocks(int64_t work, int block)
{
    const int64_t want = (work + block - 1) / block;
    const int64_t cap = (int64_t)device_cu_count() * 32;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

hipError_t launch_p2g_direct(int dim, int n, int frac_bits, const Fields &p, const uint32_t *order, RangesF r,
                             int64_t *grid, uint32_t *status, hipStream_t s)
{
    if (p.n == 0)
        return hipSuccess;
    const float nf = (float)n, dx = 1.0f / (float)n, last = (float)(n - 3), S = ldexpf(1.0f, frac_bits);
    const int blocks = grid_blocks(p.n, 256);
    if (dim == 3)
        hipLaunchKernelGGL(p2g_direct_kernel<3>, dim3(blocks), dim3(256), 0, s, p, order, n, nf, dx, last, S, r,
                           grid, status);
    else
        hipLaunchKernelGGL(p2g_direct_kernel<2>, dim3(blocks), dim3(256), 0, s, p, order, n, nf, dx, last, S, r,
                           grid, status);
    return hipGetLastError();
}

hipError_t launch_p2g_tiled(int dim, int n, int frac_bits, const BinView &b, int64_t *grid, uint32_t *status,
                            hipStream_t s)
{
    TiledArgs a;
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
    a.grid = grid;
    a.status = status;
    hipLaunchKernelGGL(reset_cursor_kernel, dim3(1), dim3(1), 0, s, a.cursor);
    int per_cu = 0;
    hipError_t e;
    if (dim == 3)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, p2g_tiled_kernel<3>, kWave, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, p2g_tiled_kernel<2>, kWave, 0);
    if (e != hipSuccess)
        return e;
    int64_t blocks = (int64_t)device_cu_count() * (per_cu > 0 ? per_cu : 1);
    if (blocks > b.max_items)
        blocks = b.max_items;
    if (blocks < 1)
        blocks = 1;
    if (dim == 3)
        hipLaunchKernelGGL(p2g_tiled_kernel<3>, dim3((unsigned)blocks), dim3(kWave), 0, s, a);
    else
        hipLaunchKernelGGL(p2g_tiled_kernel<2>, dim3((unsigned)blocks), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_p2g_cic_split(int64_t n, const int32_t *X, const int32_t *m, const int32_t *vel,
                                const uint32_t *order, int cells, int64_t *grid, uint32_t *status, hipStream_t s)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(p2g_cic_split_kernel, dim3(grid_blocks(n, 256)), dim3(256), 0, s, n, X, m, vel, order, cells,
                       grid, status);
    return hipGetLastError();
}

}  // namespace mpmk
