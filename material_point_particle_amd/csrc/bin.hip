// bin.hip -- counting sort of particles into tiles of 4^dim cells (gfx950).
//
// "Particle worlds, part 3" (steps 3 and 4): a histogram of cell numbers, an
// exclusive prefix sum, and a scatter of each particle to its slot; the
// implementation page's section 2.1 bins particles into tiles every substep
// and builds an index table so the particle arrays themselves never move.
//
// Passes (all on the caller's stream, no host synchronisation):
//   1. count    one thread per particle: base cell -> tile-major cell key;
//               atomic increment of the cell's counter returns the particle's
//               arrival rank inside the cell.
//   2. scan     exclusive prefix sum of the cell counters, each rounded up to
//               a multiple of kGroup (three phases: per-block sums, one block
//               scans the sums, per-block rescan).
//   3. layout   per tile: rows of kRowSlots record slots (one group of kGroup
//               same-cell records per lane), full P2G work items of
//               kRowsPerItem rows and a partial last item; rows and full items
//               prefix-summed over tiles, partial items counting-sorted by
//               size (largest first).
//   4. items    the (tile, first row) of every work item, alternately from the
//               large and the small end of the size order; and a compact
//               (first position, rows, first row) record per tile.
//   5. scatter  one thread per particle: its slot in the tile's grouped,
//               transposed layout (group g of a tile with R rows sits in lane
//               g / R of row g % R); the particle's slot and a record of
//               the particle's fields (x, v, C, m: 64 bytes in 3D) are written
//               there, so each scattered write is one whole record.
//   6. pad      one thread per cell: zero-mass records complete the cell's
//               last group.
// Arrival ranks depend on scheduling, so slot contents differ between runs;
// every group holds kGroup records of one cell, which is all P2G needs.
#include "common.hpp"

namespace mpmk {
namespace {

constexpr int kScanBlock = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanBlock * kScanItems;

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

// Exclusive scan across the block of one value per thread; returns the
// exclusive prefix and writes the block total to *total.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *total)
{
    __shared__ uint32_t wsum[BLOCK / kWave];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1)
        wsum[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        uint32_t w = lane < BLOCK / kWave ? wsum[lane] : 0u;
        const uint32_t winc = wave_inclusive_scan(w);
        if (lane < BLOCK / kWave)
            wsum[lane] = winc - w;
        if (lane == kWave - 1)
            *total = winc;
    }
    __syncthreads();
    const uint32_t r = wsum[wid] + inc - v;
    __syncthreads();
    return r;
}

// The scans read each counter rounded up to a multiple of ROUND (1 or kGroup).
template <int ROUND>
__device__ __forceinline__ uint32_t scan_load(const uint32_t *in, int64_t k)
{
    const uint32_t v = in[k];
    return ROUND == 1 ? v : (v + (ROUND - 1)) / ROUND * ROUND;
}

template <int ROUND>
__global__ void __launch_bounds__(kScanBlock) scan_reduce_kernel(const uint32_t *__restrict__ in, int64_t len,
                                                                 uint32_t *__restrict__ partial)
{
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    uint32_t s = 0;
    for (int i = threadIdx.x; i < kScanTile; i += kScanBlock) {
        const int64_t k = base + i;
        if (k < len)
            s += scan_load<ROUND>(in, k);
    }
    __shared__ uint32_t tot;
    (void)block_exclusive_scan<kScanBlock>(s, &tot);
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.x] = tot;
}

// One block: exclusive scan of the per-block sums in place; grand total to *total.
__global__ void __launch_bounds__(1024) scan_partials_kernel(uint32_t *__restrict__ partial, int64_t nblocks,
                                                             uint32_t *__restrict__ total)
{
    __shared__ uint32_t chunk_total;
    uint32_t carry = 0;
    for (int64_t base = 0; base < nblocks; base += 1024) {
        const int64_t k = base + threadIdx.x;
        const uint32_t v = k < nblocks ? partial[k] : 0u;
        const uint32_t ex = block_exclusive_scan<1024>(v, &chunk_total);
        if (k < nblocks)
            partial[k] = carry + ex;
        __syncthreads();
        carry += chunk_total;
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *total = carry;
}

template <int ROUND>
__global__ void __launch_bounds__(kScanBlock) scan_final_kernel(const uint32_t *__restrict__ in, int64_t len,
                                                                const uint32_t *__restrict__ partial,
                                                                uint32_t *__restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    const bool full = (int64_t)(blockIdx.x + 1) * kScanTile <= len;   // uniform across the block
    uint32_t v[kScanItems];
    uint32_t s = 0;
    if (full) {                      // 16 consecutive words per thread as four 16-byte loads
        const uint4 *src = reinterpret_cast<const uint4 *>(in + base);
#pragma unroll
        for (int q = 0; q < kScanItems / 4; ++q) {
            const uint4 t = src[q];
            v[4 * q] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            if (ROUND != 1)
                v[i] = (v[i] + (ROUND - 1)) / ROUND * ROUND;
            s += v[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            const int64_t k = base + i;
            v[i] = k < len ? scan_load<ROUND>(in, k) : 0u;
            s += v[i];
        }
    }
    __shared__ uint32_t tot;
    uint32_t run = block_exclusive_scan<kScanBlock>(s, &tot) + partial[blockIdx.x];
    if (full) {
        uint32_t o[kScanItems];
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            o[i] = run;
            run += v[i];
        }
        uint4 *dst = reinterpret_cast<uint4 *>(out + base);
#pragma unroll
        for (int q = 0; q < kScanItems / 4; ++q)
            dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            const int64_t k = base + i;
            if (k < len)
                out[k] = run;
            run += v[i];
        }
    }
}

__global__ void fill_u32_kernel(uint32_t *__restrict__ p, int64_t count, uint32_t value)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// out[0..len] = exclusive prefix sum of in[0..len) (each value rounded up to a
// multiple of ROUND), out[len] = total.  scratch holds ceil(len / kScanTile) words.
template <int ROUND>
hipError_t exclusive_scan(const uint32_t *in, int64_t len, uint32_t *out, uint32_t *scratch, hipStream_t s)
{
    const int64_t nb = (len + kScanTile - 1) / kScanTile;
    if (nb == 0) {
        hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, out, (int64_t)1, 0u);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(scan_reduce_kernel<ROUND>, dim3((unsigned)nb), dim3(kScanBlock), 0, s, in, len, scratch);
    hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(1024), 0, s, scratch, nb, out + len);
    hipLaunchKernelGGL(scan_final_kernel<ROUND>, dim3((unsigned)nb), dim3(kScanBlock), 0, s, in, len, scratch, out);
    return hipGetLastError();
}

// Pass 1: cell key (tile, then the cell's local number, see tile_local) from
// the position only; particles whose stencil leaves the
// grid are counted and not binned.  The attribute range check happens in the
// scatter pass, which reads the attributes anyway.
//
// Blocks visit 256-particle chunks in the order chunk = (i * stride) mod
// chunks (stride a prime not dividing the chunk count), so the blocks that
// run at the same time hold particles from all over the caller's array.
// Input arrays often list particles region by region (a generator filling one
// blob or block after another); visiting them in order would aim every
// concurrent atomic at the few cells of one region and serialise them.
template <int DIM>
__global__ void __launch_bounds__(256) bin_count_kernel(Fields f, float nf, float dx, float last_base, int ntx,
                                                         uint32_t *__restrict__ cell_count,
                                                         uint32_t *__restrict__ key_out,
                                                         uint32_t *__restrict__ rank_out,
                                                         uint32_t *__restrict__ status, uint32_t *__restrict__ meta,
                                                         int64_t chunks, int64_t stride)
{
    constexpr int per_tile = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    uint32_t binned = 0;
    for (int64_t i = blockIdx.x; i < chunks; i += gridDim.x) {
        const int64_t p = ((i * stride) % chunks) * 256 + threadIdx.x;
        if (p >= f.n)
            continue;
        bool dom = true;
        int base[DIM];
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            Axis ax;
            dom = axis_stencil(f.x[e * f.n + p], nf, dx, last_base, ax) && dom;
            base[e] = ax.base;
        }
        wave_count(!dom, &status[0]);
        binned += dom ? 1u : 0u;
        uint32_t key = kEmpty, rank = 0;
        if (dom) {
            uint32_t t = 0, l[DIM];
#pragma unroll
            for (int e = DIM - 1; e >= 0; --e) {
                t = t * (uint32_t)ntx + (uint32_t)(base[e] / kTile);
                l[e] = (uint32_t)(base[e] % kTile);
            }
            key = t * per_tile + tile_local<DIM>(l);
            rank = atomicAdd(&cell_count[key], 1u);
        }
        key_out[p] = key;
        rank_out[p] = rank;
    }
    // one atomic per block for the binned-particle total (a per-wave atomic on
    // one address from every wave of the grid would serialise)
    __shared__ uint32_t total;
    (void)block_exclusive_scan<256>(binned, &total);
    if (threadIdx.x == 0 && total != 0u)
        atomicAdd(&meta[2], total);
}

// Pass 3: per tile, rows of kRowSlots record slots (one group of kGroup
// records per lane), its number of full work items (kRowsPerItem rows each)
// and the size of its last, partial item.  P2G hands items out dynamically;
// the items are ordered by size (all full items, then the partial items by
// decreasing size) and handed out alternately from both ends of that order
// (see items_kernel).  The partial sizes are counting-sorted: one block of 256 tiles counts them per
// size in LDS (the returned count is the tile's rank within the block) and
// writes its histogram, size-major, for a prefix sum.  One thread per tile.
template <int DIM>
__global__ void __launch_bounds__(256) tile_layout_kernel(const uint32_t *__restrict__ cell_start, int64_t n_tiles,
                                                           uint32_t *__restrict__ tile_rows,
                                                           uint32_t *__restrict__ tile_full,
                                                           uint32_t *__restrict__ tile_part,
                                                           uint32_t *__restrict__ item_hist)
{
    constexpr int per_tile = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    __shared__ uint32_t hist[kRowsPerItem];
    if (threadIdx.x < kRowsPerItem)
        hist[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t part = 0, rank = 0;
    if (t < n_tiles) {
        const uint32_t padded = cell_start[(t + 1) * per_tile] - cell_start[t * per_tile];
        const uint32_t rows = (padded + kRowSlots - 1) / kRowSlots;
        part = rows % kRowsPerItem;
        tile_rows[t] = rows;
        tile_full[t] = rows / kRowsPerItem;
        if (part != 0u)
            rank = atomicAdd(&hist[part], 1u);
        tile_part[t] = (part << 16) | rank;
    }
    __syncthreads();
    // row (kRowsPerItem - 1 - size) of the size-major histogram: largest size first
    if (threadIdx.x >= 1 && threadIdx.x < kRowsPerItem)
        item_hist[(int64_t)(kRowsPerItem - 1 - threadIdx.x) * gridDim.x + blockIdx.x] = hist[threadIdx.x];
}

// Pass 4: the work items of each tile, and a compact per-tile record
// (padded first position, rows, first row) for the scatter pass.
template <int DIM>
__global__ void __launch_bounds__(256) items_kernel(const uint32_t *__restrict__ tile_rows,
                                                     const uint32_t *__restrict__ tile_full,
                                                     const uint32_t *__restrict__ tile_part,
                                                     const uint32_t *__restrict__ full_start,
                                                     const uint32_t *__restrict__ hist_start,
                                                     const uint32_t *__restrict__ tile_row_start,
                                                     const uint32_t *__restrict__ cell_start, int64_t n_tiles,
                                                     int64_t layout_blocks, uint4 *__restrict__ items,
                                                     uint4 *__restrict__ tile_info)
{
    constexpr int per_tile = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    const uint32_t n_full = full_start[n_tiles];
    const uint32_t total = n_full + hist_start[(int64_t)(kRowsPerItem - 1) * layout_blocks];
    // p is an item's position in the size-sorted list; the items are handed
    // out alternately from its two ends (largest, smallest, second largest,
    // ...), so long and short items run side by side on every CU and the last
    // items handed out are short.
    auto place = [&](uint32_t p) { return p < (total + 1) / 2 ? 2 * p : 2 * (total - 1 - p) + 1; };
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n_tiles; t += (int64_t)gridDim.x * blockDim.x) {
        // one 16-byte record per item: tile, first row | end row << 16,
        // groups of the tile, first row of the tile in the binned copy
        const uint32_t k = tile_full[t], s0 = full_start[t], rows = tile_rows[t];
        const uint32_t groups = (cell_start[(t + 1) * per_tile] - cell_start[t * per_tile]) / kGroup;
        const uint32_t base = tile_row_start[t];
        for (uint32_t c = 0; c < k; ++c)
            items[place(s0 + c)] = make_uint4((uint32_t)t, (c * kRowsPerItem) | ((c + 1) * kRowsPerItem << 16),
                                              groups, base);
        const uint32_t part = tile_part[t] >> 16;
        if (part != 0u) {
            const uint32_t q = place(n_full + hist_start[(int64_t)(kRowsPerItem - 1 - part) * layout_blocks + t / 256] +
                                     (tile_part[t] & 0xFFFFu));
            items[q] = make_uint4((uint32_t)t, (k * kRowsPerItem) | (rows << 16), groups, base);
        }
        tile_info[t] = make_uint4(cell_start[t * per_tile], tile_rows[t], tile_row_start[t], 0u);
    }
}

__global__ void meta_kernel(const uint32_t *__restrict__ full_start, const uint32_t *__restrict__ hist_start,
                            int64_t hist_len, const uint32_t *__restrict__ tile_row_start,
                            const uint32_t *__restrict__ cell_start, int64_t n_tiles, int64_t n_cells,
                            uint32_t *__restrict__ meta)
{
    meta[0] = full_start[n_tiles] + hist_start[hist_len];
    meta[1] = tile_row_start[n_tiles];
    meta[3] = 0u;
    meta[4] = cell_start[n_cells];
}

// Record slot of padded cell-sorted position s in a tile with `rows` rows:
// group g = s / kGroup sits in lane g / rows of row g % rows, element s % kGroup.
__device__ __forceinline__ int64_t slot_of(uint32_t row_start, uint32_t rows, uint32_t s)
{
    const uint32_t g = s / kGroup;
    return ((int64_t)row_start + g % rows) * kRowSlots + (int64_t)(s % kGroup) * kWave + g / rows;
}

// Pass 5: place each binned particle's record.  Particles outside the
// declared ranges are counted and written with zero mass, velocity and affine
// matrix: they contribute nothing, as if skipped.
template <int DIM>
__global__ void __launch_bounds__(256) bin_scatter_kernel(Fields f, RangesF r, const uint32_t *__restrict__ key_in,
                                                           const uint32_t *__restrict__ rank_in,
                                                           const uint32_t *__restrict__ cell_start,
                                                           const uint4 *__restrict__ tile_info,
                                                           uint32_t *__restrict__ slot_out,
                                                           float *__restrict__ sorted, uint32_t *__restrict__ status)
{
    constexpr int per_tile = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    constexpr int R = rec_floats<DIM>();
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < f.n; p += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t key = key_in[p];
        const bool binned = key != kEmpty;
        float rec[R];
        bool rng = false;
        if (binned) {
            int fi = 0;
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                rec[fi++] = f.x[e * f.n + p];
            rng = fabsf(f.m[p]) <= r.max_mass;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                rec[fi] = f.v[e * f.n + p];
                rng = rng && fabsf(rec[fi]) <= r.max_speed;
                ++fi;
            }
#pragma unroll
            for (int k = 0; k < DIM * DIM; ++k) {
                rec[fi] = f.C ? f.C[k * f.n + p] : 0.0f;
                rng = rng && fabsf(rec[fi]) <= r.max_affine;
                ++fi;
            }
            rec[fi++] = f.m[p];
#pragma unroll
            for (; fi < R; ++fi)
                rec[fi] = 0.0f;
            if (!rng) {
#pragma unroll
                for (int k = DIM; k < R; ++k)
                    rec[k] = 0.0f;
            }
        }
        wave_count(binned && !rng, &status[1]);
        if (!binned) {
            slot_out[p] = kEmpty;
            continue;
        }
        const uint4 ti = tile_info[key / per_tile];           // (first, rows, row_start, -)
        const uint32_t s = cell_start[key] - ti.x + rank_in[p];
        const int64_t slot = slot_of(ti.z, ti.y, s);
        slot_out[p] = (uint32_t)slot;
        float4 *dst = reinterpret_cast<float4 *>(sorted + slot * R);
#pragma unroll
        for (int q = 0; q < R / 4; ++q)
            dst[q] = make_float4(rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3]);
    }
}

// Pass 6: pad records.  A cell whose count is not a multiple of kGroup gets
// zero-mass records at its centre (g = base + 1 on every axis, which lies in
// the same base cell) in its remaining group positions; the transfer turns
// them into exact zero contributions.
template <int DIM>
__global__ void __launch_bounds__(256) bin_pad_kernel(const uint32_t *__restrict__ cell_count,
                                                       const uint32_t *__restrict__ cell_start,
                                                       const uint4 *__restrict__ tile_info, int64_t n_cells, int ntx,
                                                       float inv_n, float *__restrict__ sorted)
{
    constexpr int per_tile = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    constexpr int R = rec_floats<DIM>();
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_cells; c += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t count = cell_count[c];
        const uint32_t rem = count % kGroup;
        if (rem == 0)
            continue;
        const uint32_t tile = (uint32_t)(c / per_tile), local = (uint32_t)(c % per_tile);
        const uint4 ti = tile_info[tile];
        float rec[R];
#pragma unroll
        for (int k = 0; k < R; ++k)
            rec[k] = 0.0f;
        uint32_t t = tile, l[DIM];
        tile_local_inverse<DIM>(local, l);
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            const uint32_t base = (t % (uint32_t)ntx) * kTile + l[e];
            rec[e] = (float)(base + 1) * inv_n;
            t /= (uint32_t)ntx;
        }
        const uint32_t s0 = cell_start[c] - ti.x + count;
        for (uint32_t s = s0; s < s0 + (kGroup - rem); ++s) {
            float4 *dst = reinterpret_cast<float4 *>(sorted + slot_of(ti.z, ti.y, s) * R);
#pragma unroll
            for (int q = 0; q < R / 4; ++q)
                dst[q] = make_float4(rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3]);
        }
    }
}

// A prime step that does not divide `chunks`, so i -> (i * step) mod chunks
// is a permutation of the chunks.
int64_t chunk_stride(int64_t chunks)
{
    const int64_t primes[] = { 7919, 104729, 1299709, 15485863 };
    for (int64_t q : primes)
        if (chunks % q != 0)
            return q % (chunks > 0 ? chunks : 1) == 0 ? 1 : q;
    return 1;
}

int blocks_for(int64_t work, int block)
{
    const int64_t want = (work + block - 1) / block;
    const int64_t cap = (int64_t)device_cu_count() * 32;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

hipError_t launch_bin(int dim, int n, const Fields &p, RangesF r, const BinView &b, uint32_t *status, hipStream_t s)
{
    const float nf = (float)n, dx = 1.0f / (float)n, last = (float)(n - 3);
    const int ntx = n / kTile;
    uint32_t *tile_rows = b.tile_tmp, *tile_items = b.tile_tmp + b.n_tiles;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks_for(b.n_cells, 256)), dim3(256), 0, s, b.cell_count, b.n_cells,
                       0u);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, b.meta, (int64_t)16, 0u);
    const int64_t chunks = (p.n + 255) / 256;
    const int64_t stride = chunk_stride(chunks);
    if (dim == 3)
        hipLaunchKernelGGL(bin_count_kernel<3>, dim3(blocks_for(p.n, 256)), dim3(256), 0, s, p, nf, dx, last, ntx,
                           b.cell_count, b.key, b.rank, status, b.meta, chunks, stride);
    else
        hipLaunchKernelGGL(bin_count_kernel<2>, dim3(blocks_for(p.n, 256)), dim3(256), 0, s, p, nf, dx, last, ntx,
                           b.cell_count, b.key, b.rank, status, b.meta, chunks, stride);
    hipError_t e = exclusive_scan<kGroup>(b.cell_count, b.n_cells, b.cell_start, b.scan_tmp, s);
    if (e != hipSuccess)
        return e;
    const int64_t lblocks = (b.n_tiles + 255) / 256;
    uint32_t *tile_part = b.tile_tmp + 2 * b.n_tiles;
    const int64_t hist_len = (kRowsPerItem - 1) * lblocks;
    if (dim == 3)
        hipLaunchKernelGGL(tile_layout_kernel<3>, dim3((unsigned)lblocks), dim3(256), 0, s, b.cell_start, b.n_tiles,
                           tile_rows, tile_items, tile_part, b.item_hist);
    else
        hipLaunchKernelGGL(tile_layout_kernel<2>, dim3((unsigned)lblocks), dim3(256), 0, s, b.cell_start, b.n_tiles,
                           tile_rows, tile_items, tile_part, b.item_hist);
    if ((e = exclusive_scan<1>(tile_rows, b.n_tiles, b.tile_row_start, b.scan_tmp, s)) != hipSuccess)
        return e;
    if ((e = exclusive_scan<1>(tile_items, b.n_tiles, b.item_start, b.scan_tmp, s)) != hipSuccess)
        return e;
    if ((e = exclusive_scan<1>(b.item_hist, hist_len, b.item_hist_start, b.scan_tmp, s)) != hipSuccess)
        return e;
    uint4 *tile_info = reinterpret_cast<uint4 *>(b.tile_info);
    if (dim == 3)
        hipLaunchKernelGGL(items_kernel<3>, dim3(blocks_for(b.n_tiles, 256)), dim3(256), 0, s, tile_rows, tile_items,
                           tile_part, b.item_start, b.item_hist_start, b.tile_row_start, b.cell_start, b.n_tiles,
                           lblocks, reinterpret_cast<uint4 *>(b.items), tile_info);
    else
        hipLaunchKernelGGL(items_kernel<2>, dim3(blocks_for(b.n_tiles, 256)), dim3(256), 0, s, tile_rows, tile_items,
                           tile_part, b.item_start, b.item_hist_start, b.tile_row_start, b.cell_start, b.n_tiles,
                           lblocks, reinterpret_cast<uint4 *>(b.items), tile_info);
    hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(1), 0, s, b.item_start, b.item_hist_start, hist_len,
                       b.tile_row_start, b.cell_start, b.n_tiles, b.n_cells, b.meta);
    if (dim == 3) {
        hipLaunchKernelGGL(bin_scatter_kernel<3>, dim3(blocks_for(p.n, 256)), dim3(256), 0, s, p, r, b.key, b.rank,
                           b.cell_start, tile_info, b.slot, b.sorted, status);
        hipLaunchKernelGGL(bin_pad_kernel<3>, dim3(blocks_for(b.n_cells, 256)), dim3(256), 0, s, b.cell_count,
                           b.cell_start, tile_info, b.n_cells, ntx, 1.0f / (float)n, b.sorted);
    } else {
        hipLaunchKernelGGL(bin_scatter_kernel<2>, dim3(blocks_for(p.n, 256)), dim3(256), 0, s, p, r, b.key, b.rank,
                           b.cell_start, tile_info, b.slot, b.sorted, status);
        hipLaunchKernelGGL(bin_pad_kernel<2>, dim3(blocks_for(b.n_cells, 256)), dim3(256), 0, s, b.cell_count,
                           b.cell_start, tile_info, b.n_cells, ntx, 1.0f / (float)n, b.sorted);
    }
    return hipGetLastError();
}

}  // namespace mpmk
