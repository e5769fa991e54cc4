// bin.hip -- counting sort of particles into tiles of 4^dim cells (gfx950).
//
// "Particle worlds, part 3" (steps 3 and 4): a histogram of keys, an
// exclusive prefix sum, and a scatter of each particle to its place; the
// implementation page's section 2.1 bins particles into tiles every substep
// and builds an index table so the particle arrays themselves never move.
// Here the particles are counting-sorted by tile; P2G sorts the cells of each
// work item on chip.
//
// Passes (all on the caller's stream, no host synchronisation):
//   1. count    blocks of up to 65,536 consecutive particles (a chunk): each
//               particle's base cell gives its tile; an LDS hash table counts
//               the chunk's particles per tile, then one global atomic per
//               (chunk, tile) reserves the chunk's run inside the tile, so a
//               particle's rank in its tile is its run's base plus its rank
//               in the chunk.
//   2. scan     exclusive prefix sum of the tile counts: each tile's first
//               record.
//   3. layout   each tile's records are cut into slices of at most
//               slice_records(), one P2G work item each; full slices counted
//               and prefix-summed over tiles, partial slices counting-sorted
//               by the rows their groups need.
//   4. items    the 16-byte record of every work item, alternately from the
//               large and the small end of the size order.
//   5. scatter  the same chunks as pass 1: each particle's 64-byte record
//               (x, v, C, m in 3D) goes to its tile's record range at its
//               rank, with the cell's local number beside it.  A chunk's
//               particles of one tile land in one contiguous run.
// Arrival ranks depend on scheduling, so record order inside a tile differs
// between runs; P2G's grid does not depend on it.
#include "common.hpp"

namespace mpmk {
namespace {

constexpr int kScanBlock = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanBlock * kScanItems;

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

// Passes 1 and 5 visit the same chunks of kBinThreads * per consecutive
// particles (per <= kMaxPer, chosen per launch so that every CU gets chunks),
// one block per chunk.
constexpr int kBinThreads = 1024;
constexpr int kMaxPer = 64;                          // a chunk holds at most 65,536 particles
constexpr int kHashBits = 11;
constexpr int kHashSlots = 1 << kHashBits;           // tiles per chunk counted in LDS
constexpr int kMaxProbes = 64;
constexpr uint32_t kLocalRank = 0x80000000u;         // rank_out holds (slot << 16) | rank in the chunk
static_assert(kBinThreads * kMaxPer <= 65536, "a rank inside the chunk must fit 16 bits");

// Tile and local cell number (see tile_local) of the particle's base cell;
// false when its stencil leaves the grid.
template <int DIM>
__device__ __forceinline__ bool particle_cell(const float *x, float nf, float dx, float last_base, int ntx,
                                              uint32_t &tile, uint32_t &local)
{
    bool dom = true;
    int base[DIM];
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        Axis ax;
        dom = axis_stencil(x[e], nf, dx, last_base, ax) && dom;
        base[e] = ax.base;
    }
    uint32_t t = 0, l[DIM];
#pragma unroll
    for (int e = DIM - 1; e >= 0; --e) {
        t = t * (uint32_t)ntx + (uint32_t)(base[e] / kTile);
        l[e] = (uint32_t)(base[e] % kTile);
    }
    tile = t;
    local = tile_local<DIM>(l);
    return dom;
}

// Pass 1.  Particles whose stencil leaves the grid are counted (status[0])
// and not binned; the attribute range check happens in pass 5, which reads
// the attributes anyway.  An LDS hash table counts the chunk's particles per
// tile; after the chunk, one global atomic per table entry reserves the
// chunk's run inside the tile, and each particle's rank becomes the run's
// base plus its rank in the chunk.  A particle whose tile finds no table
// entry within kMaxProbes probes takes a rank of its own with a global atomic.
// Input that lists particles region by region (as generators and simulations
// usually leave it) touches few tiles per chunk, so the global atomics number
// a few hundred per chunk, and each tile's records from one chunk form one
// contiguous run for pass 5 to write.  Inside a run the records keep their
// arrival order, so records written close together in time are neighbours in
// memory.
template <int DIM>
__global__ void __launch_bounds__(kBinThreads) bin_tile_count_kernel(Fields f, float nf, float dx, float last_base,
                                                                      int ntx, int64_t chunks, int per,
                                                                      uint32_t *__restrict__ tile_count,
                                                                      uint32_t *__restrict__ rank_out,
                                                                      uint32_t *__restrict__ status,
                                                                      uint32_t *__restrict__ meta)
{
    __shared__ uint32_t hkey[kHashSlots];
    __shared__ uint32_t hval[kHashSlots];     // count in the chunk, then the chunk's base in the tile
    for (int e = threadIdx.x; e < kHashSlots; e += kBinThreads) {
        hkey[e] = kEmpty;
        hval[e] = 0u;
    }
    __syncthreads();
    uint32_t binned = 0;
    const int64_t chunk = (int64_t)kBinThreads * per;
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const int64_t p0 = c * chunk + threadIdx.x;
        for (int k0 = 0; k0 < per; k0 += 4) {
            float xs[4][DIM];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = p0 + (int64_t)(k0 + j) * kBinThreads;
#pragma unroll
                for (int e = 0; e < DIM; ++e)
                    xs[j][e] = (k0 + j < per && p < f.n) ? f.x[e * f.n + p] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = p0 + (int64_t)(k0 + j) * kBinThreads;
                const bool live = k0 + j < per && p < f.n;
                uint32_t t = 0, l = 0;
                const bool dom = live && particle_cell<DIM>(xs[j], nf, dx, last_base, ntx, t, l);
                wave_count(live && !dom, &status[0]);
                if (!live)
                    continue;
                uint32_t v = 0u;
                if (dom) {
                    uint32_t h = (t * 0x9E3779B1u) >> (32 - kHashBits);
                    bool found = false;
                    for (int probe = 0; probe < kMaxProbes; ++probe) {
                        const uint32_t old = atomicCAS(&hkey[h], kEmpty, t);
                        if (old == kEmpty || old == t) {
                            found = true;
                            break;
                        }
                        h = (h + 1u) & (kHashSlots - 1);
                    }
                    v = found ? kLocalRank | (h << 16) | atomicAdd(&hval[h], 1u) : atomicAdd(&tile_count[t], 1u);
                    ++binned;
                }
                rank_out[p] = v;
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < kHashSlots; e += kBinThreads) {
            const uint32_t key = hkey[e];
            if (key != kEmpty)
                hval[e] = atomicAdd(&tile_count[key], hval[e]);
        }
        __syncthreads();
        for (int k = 0; k < per; ++k) {            // the thread's own writes above: no fence needed
            const int64_t p = p0 + (int64_t)k * kBinThreads;
            if (p >= f.n)
                break;
            const uint32_t v = rank_out[p];
            if (v & kLocalRank)
                rank_out[p] = hval[(v >> 16) & (kHashSlots - 1)] + (v & 0xFFFFu);
        }
        __syncthreads();
        for (int e = threadIdx.x; e < kHashSlots; e += kBinThreads) {
            hkey[e] = kEmpty;
            hval[e] = 0u;
        }
        __syncthreads();
    }
    // one atomic per block for the binned-particle total (a per-wave atomic on
    // one address from every wave of the grid would serialise)
    __shared__ uint32_t total;
    (void)block_exclusive_scan<kBinThreads>(binned, &total);
    if (threadIdx.x == 0 && total != 0u)
        atomicAdd(&meta[2], total);
}

// Pass 3: each tile's records are cut into slices of slice_records() (the
// last one shorter), one P2G work item each; a slice's groups fill at most
// kRowsPerItem rows.  Per tile: its full slices and the rows of its last,
// partial slice.  P2G hands items out dynamically; the items are
// ordered by size (all full slices, then the partial slices by decreasing
// rows) and handed out alternately from both ends of that order (see
// items_kernel).  The partial slices are counting-sorted by rows: one block of
// 256 tiles counts them per row count in LDS (the returned count is the
// tile's rank within the block) and writes its histogram, size-major, for a
// prefix sum.  One thread per tile.
template <int DIM>
__global__ void __launch_bounds__(256) tile_layout_kernel(const uint32_t *__restrict__ tile_count, int64_t n_tiles,
                                                           uint32_t *__restrict__ tile_full,
                                                           uint32_t *__restrict__ tile_part,
                                                           uint32_t *__restrict__ item_hist)
{
    constexpr uint32_t S = slice_records<DIM>();
    __shared__ uint32_t hist[kRowsPerItem + 1];
    if (threadIdx.x <= kRowsPerItem)
        hist[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n_tiles) {
        const uint32_t c = tile_count[t];
        const uint32_t full = c / S, rem = c % S;
        const uint32_t part = rem != 0u ? rows_bound<DIM>(rem) : 0u;      // 1 .. kRowsPerItem
        uint32_t rank = 0;
        tile_full[t] = full;
        if (part != 0u)
            rank = atomicAdd(&hist[part], 1u);
        tile_part[t] = (part << 16) | rank;
    }
    __syncthreads();
    // row (kRowsPerItem - rows) of the size-major histogram: largest first
    if (threadIdx.x >= 1 && threadIdx.x <= kRowsPerItem)
        item_hist[(int64_t)(kRowsPerItem - threadIdx.x) * gridDim.x + blockIdx.x] = hist[threadIdx.x];
}

// Pass 4: the work items of each tile.  One 16-byte record per item: tile,
// first record, records, 0.
template <int DIM>
__global__ void __launch_bounds__(256) items_kernel(const uint32_t *__restrict__ tile_full,
                                                     const uint32_t *__restrict__ tile_part,
                                                     const uint32_t *__restrict__ full_start,
                                                     const uint32_t *__restrict__ hist_start,
                                                     const uint32_t *__restrict__ tile_start, int64_t n_tiles,
                                                     int64_t layout_blocks, uint4 *__restrict__ items)
{
    constexpr uint32_t S = slice_records<DIM>();
    const uint32_t n_full = full_start[n_tiles];
    const uint32_t total = n_full + hist_start[(int64_t)kRowsPerItem * layout_blocks];
    // p is an item's position in the size-sorted list; the items are handed
    // out alternately from its two ends (largest, smallest, second largest,
    // ...), so long and short items run side by side on every CU and the last
    // items handed out are short.
    auto place = [&](uint32_t p) { return p < (total + 1) / 2 ? 2 * p : 2 * (total - 1 - p) + 1; };
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n_tiles; t += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t k = tile_full[t], s0 = full_start[t];
        const uint32_t c0 = tile_start[t], count = tile_start[t + 1] - c0;
        for (uint32_t c = 0; c < k; ++c)
            items[place(s0 + c)] = make_uint4((uint32_t)t, c0 + c * S, S, 0u);
        const uint32_t part = tile_part[t] >> 16;
        if (part != 0u) {
            const uint32_t q = place(n_full + hist_start[(int64_t)(kRowsPerItem - part) * layout_blocks + t / 256] +
                                     (tile_part[t] & 0xFFFFu));
            items[q] = make_uint4((uint32_t)t, c0 + k * S, count - k * S, 0u);
        }
    }
}

// meta: [0] work items, [3] P2G's work cursor ([2], the binned particles, is
// added to by pass 1).
__global__ void meta_kernel(const uint32_t *__restrict__ full_start, const uint32_t *__restrict__ hist_start,
                            int64_t hist_len, int64_t n_tiles, uint32_t *__restrict__ meta)
{
    meta[0] = full_start[n_tiles] + hist_start[hist_len];
    meta[3] = 0u;
}

// Pass 5: each binned particle's record at its tile's first record plus its
// rank.  Particles outside the declared ranges are counted and written with
// zero mass, velocity and affine matrix: they contribute nothing, as if
// skipped.  Each thread loads two particles before writing either, so that
// twice the loads are in flight.  Every lane of a wavefront runs the same
// number of iterations, so all of them reach write_records's exchanges.
template <int DIM>
__device__ __forceinline__ void load_record(const Fields &f, int64_t p, float *rec)
{
    constexpr int R = rec_floats<DIM>();
    int fi = 0;
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        rec[fi++] = f.x[e * f.n + p];
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        rec[fi++] = f.v[e * f.n + p];
#pragma unroll
    for (int q = 0; q < DIM * DIM; ++q)
        rec[fi++] = f.C ? f.C[q * f.n + p] : 0.0f;
    rec[fi++] = f.m[p];
#pragma unroll
    for (; fi < R; ++fi)
        rec[fi] = 0.0f;
}

// Range check and destination of one loaded record: its index in the binned
// copy, or kEmpty when the particle is not binned.
template <int DIM>
__device__ __forceinline__ uint32_t place_record(const Fields &f, RangesF r, float nf, float dx, float last_base,
                                                 int ntx, int64_t p, float *rec,
                                                 const uint32_t *__restrict__ rank_in,
                                                 const uint32_t *__restrict__ tile_start,
                                                 uint32_t *__restrict__ slot_out, uint8_t *__restrict__ cell_key,
                                                 uint32_t *__restrict__ status)
{
    constexpr int R = rec_floats<DIM>();
    uint32_t t, l;
    if (!particle_cell<DIM>(rec, nf, dx, last_base, ntx, t, l)) {
        slot_out[p] = kEmpty;
        return kEmpty;
    }
    bool rng = fabsf(rec[2 * DIM + DIM * DIM]) <= r.max_mass;
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        rng = rng && fabsf(rec[DIM + e]) <= r.max_speed;
#pragma unroll
    for (int q = 0; q < DIM * DIM; ++q)
        rng = rng && fabsf(rec[2 * DIM + q]) <= r.max_affine;
    wave_count(!rng, &status[1]);
    if (!rng) {
#pragma unroll
        for (int q = DIM; q < R; ++q)
            rec[q] = 0.0f;
    }
    const uint32_t pos = tile_start[t] + rank_in[p];
    slot_out[p] = pos;
    cell_key[pos] = (uint8_t)l;
    return pos;
}

// Writes the wavefront's 64 records (one per lane, destination pos or kEmpty).
// In 3D a record is four 16-byte pieces; the records pass through LDS so that
// the four lanes of a quad write one record's pieces with one instruction:
// each store covers 16 whole 64-byte records instead of one piece of 64
// records, a quarter of the memory requests.  Piece q of lane L's record sits
// in slot (q + L + L / 4) mod 4 of its 64 bytes, so that eight consecutive
// lanes' 16-byte accesses fall in distinct LDS banks on both sides.
template <int DIM>
__device__ __forceinline__ void write_records(const float *rec, uint32_t pos, float4 *stage, uint32_t *spos,
                                              float *__restrict__ sorted)
{
    constexpr int R = rec_floats<DIM>();
    const int lane = threadIdx.x % kWave;
    if constexpr (DIM == 3) {
        static_assert(R == 16, "a 3D record is four float4 pieces");
#pragma unroll
        for (int q = 0; q < 4; ++q)
            stage[lane * 4 + ((q + lane + (lane >> 2)) & 3)] =
                make_float4(rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3]);
        spos[lane] = pos;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int src = 16 * i + (lane >> 2), piece = lane & 3;
            const uint32_t d = spos[src];
            const float4 v = stage[src * 4 + ((piece + src + (src >> 2)) & 3)];
            if (d != kEmpty)
                reinterpret_cast<float4 *>(sorted + (int64_t)d * R)[piece] = v;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        (void)stage;
        (void)spos;
        if (pos != kEmpty) {
            float4 *dst = reinterpret_cast<float4 *>(sorted + (int64_t)pos * R);
#pragma unroll
            for (int q = 0; q < R / 4; ++q)
                dst[q] = make_float4(rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3]);
        }
    }
}

template <int DIM>
__global__ void __launch_bounds__(kBinThreads) bin_scatter_kernel(Fields f, RangesF r, float nf, float dx,
                                                                   float last_base, int ntx, int64_t chunks, int per,
                                                                   const uint32_t *__restrict__ rank_in,
                                                                   const uint32_t *__restrict__ tile_start,
                                                                   uint32_t *__restrict__ slot_out,
                                                                   uint8_t *__restrict__ cell_key,
                                                                   float *__restrict__ sorted,
                                                                   uint32_t *__restrict__ status)
{
    constexpr int R = rec_floats<DIM>();
    constexpr int kWaves = kBinThreads / kWave;
    __shared__ float4 stage[DIM == 3 ? kWaves * kWave * 4 : 1];
    __shared__ uint32_t spos[DIM == 3 ? kWaves * kWave : 1];
    const int w = threadIdx.x / kWave;
    float4 *my_stage = DIM == 3 ? stage + w * kWave * 4 : stage;
    uint32_t *my_spos = DIM == 3 ? spos + w * kWave : spos;
    const int64_t chunk = (int64_t)kBinThreads * per;
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        for (int k = 0; k < per; k += 2) {              // uniform trip count: every lane reaches the exchanges
            const int64_t pa = c * chunk + (int64_t)k * kBinThreads + threadIdx.x;
            const int64_t pb = pa + kBinThreads;
            const bool la = pa < f.n, lb = k + 1 < per && pb < f.n;
            float ra[R], rb[R];
            if (la)
                load_record<DIM>(f, pa, ra);
            if (lb)
                load_record<DIM>(f, pb, rb);
            uint32_t da = kEmpty, db = kEmpty;
            if (la)
                da = place_record<DIM>(f, r, nf, dx, last_base, ntx, pa, ra, rank_in, tile_start, slot_out, cell_key,
                                       status);
            if (lb)
                db = place_record<DIM>(f, r, nf, dx, last_base, ntx, pb, rb, rank_in, tile_start, slot_out, cell_key,
                                       status);
            write_records<DIM>(ra, da, my_stage, my_spos, sorted);
            write_records<DIM>(rb, db, my_stage, my_spos, sorted);
        }
    }
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
    uint32_t *tile_items = b.tile_tmp, *tile_part = b.tile_tmp + b.n_tiles;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks_for(b.n_tiles, 256)), dim3(256), 0, s, b.tile_count, b.n_tiles,
                       0u);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, s, b.meta, (int64_t)16, 0u);
    // particles per thread of a chunk: enough chunks for two blocks per CU, at most kMaxPer
    const int64_t span = (int64_t)kBinThreads * device_cu_count() * 2;
    int64_t per = (p.n + span - 1) / span;
    per = per < 4 ? 4 : (per > kMaxPer ? kMaxPer : per);
    const int64_t chunks = (p.n + kBinThreads * per - 1) / (kBinThreads * per);
    const unsigned cblocks = (unsigned)(chunks < (int64_t)device_cu_count() * 2 ? chunks : device_cu_count() * 2);
    if (chunks > 0) {
        if (dim == 3)
            hipLaunchKernelGGL(bin_tile_count_kernel<3>, dim3(cblocks), dim3(kBinThreads), 0, s, p, nf, dx, last, ntx,
                               chunks, (int)per, b.tile_count, b.rank, status, b.meta);
        else
            hipLaunchKernelGGL(bin_tile_count_kernel<2>, dim3(cblocks), dim3(kBinThreads), 0, s, p, nf, dx, last, ntx,
                               chunks, (int)per, b.tile_count, b.rank, status, b.meta);
    }
    hipError_t e = exclusive_scan<1>(b.tile_count, b.n_tiles, b.tile_start, b.scan_tmp, s);
    if (e != hipSuccess)
        return e;
    const int64_t lblocks = (b.n_tiles + 255) / 256;
    const int64_t hist_len = kRowsPerItem * lblocks;
    if (dim == 3)
        hipLaunchKernelGGL(tile_layout_kernel<3>, dim3((unsigned)lblocks), dim3(256), 0, s, b.tile_count, b.n_tiles,
                           tile_items, tile_part, b.item_hist);
    else
        hipLaunchKernelGGL(tile_layout_kernel<2>, dim3((unsigned)lblocks), dim3(256), 0, s, b.tile_count, b.n_tiles,
                           tile_items, tile_part, b.item_hist);
    if ((e = exclusive_scan<1>(tile_items, b.n_tiles, b.item_start, b.scan_tmp, s)) != hipSuccess)
        return e;
    if ((e = exclusive_scan<1>(b.item_hist, hist_len, b.item_hist_start, b.scan_tmp, s)) != hipSuccess)
        return e;
    uint4 *items = reinterpret_cast<uint4 *>(b.items);
    if (dim == 3)
        hipLaunchKernelGGL(items_kernel<3>, dim3(blocks_for(b.n_tiles, 256)), dim3(256), 0, s, tile_items, tile_part,
                           b.item_start, b.item_hist_start, b.tile_start, b.n_tiles, lblocks, items);
    else
        hipLaunchKernelGGL(items_kernel<2>, dim3(blocks_for(b.n_tiles, 256)), dim3(256), 0, s, tile_items, tile_part,
                           b.item_start, b.item_hist_start, b.tile_start, b.n_tiles, lblocks, items);
    hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(1), 0, s, b.item_start, b.item_hist_start, hist_len, b.n_tiles,
                       b.meta);
    const unsigned sblocks = (unsigned)(chunks < (int64_t)device_cu_count() * 8 ? chunks : device_cu_count() * 8);
    if (chunks > 0) {
        if (dim == 3)
            hipLaunchKernelGGL(bin_scatter_kernel<3>, dim3(sblocks), dim3(kBinThreads), 0, s, p, r, nf, dx, last, ntx,
                               chunks, (int)per, b.rank, b.tile_start, b.slot, b.cell_key, b.sorted, status);
        else
            hipLaunchKernelGGL(bin_scatter_kernel<2>, dim3(sblocks), dim3(kBinThreads), 0, s, p, r, nf, dx, last, ntx,
                               chunks, (int)per, b.rank, b.tile_start, b.slot, b.cell_key, b.sorted, status);
    }
    return hipGetLastError();
}

}  // namespace mpmk
