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
//   1. count    blocks of up to 32,768 consecutive particles (a chunk): each
//               particle's base cell gives its tile; an LDS hash table counts
//               the chunk's particles per tile, then one global atomic per
//               (chunk, tile) reserves the chunk's run inside the tile, so a
//               particle's rank in its tile is its run's base plus its rank
//               in the chunk.  The table has room for every tile a chunk of
//               particles in any order touches on the workloads here, so
//               input order changes only the number of runs.
//   2-4. plan   each tile's first record (prefix sum of the counts) and its
//               work items: the tile's records cut into slices of at most
//               slice_records(), listed by size (full slices, then partial
//               slices counting-sorted by the rows their groups need) and
//               handed out alternately from the two ends of that list.
//   5. scatter  each particle's 64-byte record (x, v, C, m in 3D) goes to
//               its tile's record range at its rank; a chunk's particles of
//               one tile land in one contiguous run.  When the count's runs
//               are long (input listed region by region) the record's cell
//               key goes beside it; when they are short (input in random
//               order) those one-byte writes would land scattered and cost
//               more than the records, so none are written and P2G reads a
//               record's cell from its position (meta[kMetaKeys] says which).
// Arrival ranks depend on scheduling, so record order inside a tile differs
// between runs; P2G's grid does not depend on it.
#include "common.hpp"

namespace mpmk {
namespace {


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

// Zeroes the tile counts and the meta words, and writes the binning's stamp.
__global__ void bin_reset_kernel(uint32_t *__restrict__ tile_count, int64_t n_tiles, uint32_t *__restrict__ meta,
                                 BinStamp stamp)
{
    const uint32_t *sw = reinterpret_cast<const uint32_t *>(&stamp);
    constexpr int kStampWords = (int)(sizeof(BinStamp) / 4);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_tiles + kMetaWords;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < n_tiles) {
            tile_count[i] = 0u;
        } else {
            const int w = (int)(i - n_tiles);
            meta[w] = (w >= kMetaStamp && w < kMetaStamp + kStampWords) ? sw[w - kMetaStamp] : 0u;
        }
    }
}

// Pass 1 visits chunks of kBinThreads * PER consecutive particles (PER a
// power of two from 4 to kMaxPer, chosen per launch so that every CU gets a
// chunk, and a template argument so that each thread's PER ranks stay in
// registers), one block per chunk and one block per CU: its hash table takes
// 128 KB of LDS.  Pass 5
// needs no chunks (it reads each particle's final rank) and visits blocks of
// consecutive particles sized for occupancy.
constexpr int kBinThreads = 1024;
constexpr int kMaxPer = 32;                          // a chunk holds at most 32,768 particles
constexpr int kHashBits = 14;
constexpr int kHashSlots = 1 << kHashBits;           // tiles per chunk counted in LDS
constexpr int kMaxProbes = 64;
constexpr int kScatterPer = 32;                      // particles per thread of a scatter block, at most
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
template <int DIM, int PER>
__global__ void __launch_bounds__(kBinThreads) bin_tile_count_kernel(Fields f, float nf, float dx, float last_base,
                                                                      int ntx, int64_t chunks,
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
    uint32_t binned = 0, runs = 0;
    static_assert(PER % 4 == 0 && PER <= kMaxPer, "particles per thread");
    const int64_t chunk = (int64_t)kBinThreads * PER;
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const int64_t p0 = c * chunk + threadIdx.x;
        // per particle k of this thread: kLocalRank | slot << 16 | rank in the
        // chunk, a final rank, or 0 when not binned; kept in registers until the
        // chunk's runs are placed
        uint32_t v[PER];
#pragma unroll
        for (int k0 = 0; k0 < PER; k0 += 4) {
            float xs[4][DIM];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = p0 + (int64_t)(k0 + j) * kBinThreads;
#pragma unroll
                for (int e = 0; e < DIM; ++e)
                    xs[j][e] = p < f.n ? f.x[e * f.n + p] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = p0 + (int64_t)(k0 + j) * kBinThreads;
                const bool live = p < f.n;
                uint32_t t = 0, l = 0;
                const bool dom = live && particle_cell<DIM>(xs[j], nf, dx, last_base, ntx, t, l);
                wave_count(live && !dom, &status[0]);
                v[k0 + j] = 0u;
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
                    v[k0 + j] = found ? kLocalRank | (h << 16) | atomicAdd(&hval[h], 1u) : atomicAdd(&tile_count[t], 1u);
                    ++binned;
                    runs += found ? 0u : 1u;                 // a particle placed on its own is a run of one
                }
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < kHashSlots; e += kBinThreads) {
            const uint32_t key = hkey[e];
            if (key != kEmpty) {
                hval[e] = atomicAdd(&tile_count[key], hval[e]);
                ++runs;
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t p = p0 + (int64_t)k * kBinThreads;
            if (p < f.n)
                rank_out[p] = (v[k] & kLocalRank) ? hval[(v[k] >> 16) & (kHashSlots - 1)] + (v[k] & 0xFFFFu) : v[k];
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
    __shared__ uint32_t total, total_runs;
    (void)block_exclusive_scan<kBinThreads>(binned, &total);
    (void)block_exclusive_scan<kBinThreads>(runs, &total_runs);
    if (threadIdx.x == 0 && total != 0u) {
        atomicAdd(&meta[kMetaBinned], total);
        atomicAdd(&meta[kMetaRuns], total_runs);
    }
}

// Passes 2-4: the work-item plan.  Each tile's records are cut into slices
// of slice_records() (the last one shorter), one P2G work item each.  Per
// tile: its first record (prefix sum of the counts), its full slices and the
// rows its last, partial slice needs.  The items are listed by size (all full
// slices, then the partial slices by decreasing rows, counting-sorted by
// class) and handed out alternately from both ends of that list (largest,
// smallest, second largest, ...), so long and short items run side by side on
// every CU and the last items handed out are short.  Blocks of kPlanTiles
// tiles: pass 2 writes each block's sums and class counts, pass 3 (one block)
// prefix-sums them, pass 4 writes the tile starts and the items.
constexpr int kPlanBlock = 256;
constexpr int kPlanPer = kPlanTiles / kPlanBlock;   // tiles per thread

// Full slices and class of a tile's last, partial slice: class r holds the
// partial slices of kRowsPerItem - r rows; kRowsPerItem means none.
template <int DIM>
__device__ __forceinline__ void tile_slices(uint32_t count, uint32_t &full, uint32_t &cls)
{
    constexpr uint32_t S = slice_records<DIM>();
    full = count / S;
    const uint32_t rem = count % S;
    cls = rem != 0u ? kRowsPerItem - rows_bound<DIM>(rem) : (uint32_t)kRowsPerItem;
}

template <int DIM>
__global__ void __launch_bounds__(kPlanBlock) plan_reduce_kernel(const uint32_t *__restrict__ tile_count,
                                                                 int64_t n_tiles, uint32_t *__restrict__ part)
{
    __shared__ uint32_t hist[kRowsPerItem];
    __shared__ uint32_t tot;
    if (threadIdx.x < kRowsPerItem)
        hist[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kPlanTiles + (int64_t)threadIdx.x * kPlanPer;
    uint32_t sc = 0, sf = 0;
#pragma unroll
    for (int i = 0; i < kPlanPer; ++i) {
        const int64_t t = base + i;
        if (t < n_tiles) {
            const uint32_t c = tile_count[t];
            uint32_t full, cls;
            tile_slices<DIM>(c, full, cls);
            sc += c;
            sf += full;
            if (cls < (uint32_t)kRowsPerItem)
                atomicAdd(&hist[cls], 1u);
        }
    }
    uint32_t *out = part + (int64_t)blockIdx.x * kPlanStride;
    (void)block_exclusive_scan<kPlanBlock>(sc, &tot);
    if (threadIdx.x == 0)
        out[0] = tot;
    __syncthreads();
    (void)block_exclusive_scan<kPlanBlock>(sf, &tot);
    if (threadIdx.x == 0)
        out[1] = tot;
    if (threadIdx.x < kRowsPerItem)
        out[2 + threadIdx.x] = hist[threadIdx.x];
}

// One block: each field of the per-block records prefix-summed over the
// blocks, in place (one wavefront per field): [0] first record, [1] first
// full slice, [2 + r] first item of class r (the classes follow all full
// slices, in class order).  Writes the total record count after the tile
// starts, the item count to meta[0], and resets P2G's work cursor.
__global__ void __launch_bounds__(1024) plan_partials_kernel(uint32_t *__restrict__ part, int64_t nblocks,
                                                             uint32_t *__restrict__ tile_start_end,
                                                             uint32_t *__restrict__ meta)
{
    constexpr int kWaves = 1024 / kWave;
    __shared__ uint32_t ftot[kPlanStride];
    __shared__ uint32_t cbase[kRowsPerItem];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int f = wave; f < kPlanStride; f += kWaves) {
        uint32_t carry = 0;
        for (int64_t base = 0; base < nblocks; base += kWave) {
            const int64_t k = base + lane;
            const uint32_t v = k < nblocks ? part[k * kPlanStride + f] : 0u;
            const uint32_t inc = wave_inclusive_scan(v);
            if (k < nblocks)
                part[k * kPlanStride + f] = carry + inc - v;
            carry += __shfl(inc, kWave - 1, kWave);
        }
        if (lane == 0)
            ftot[f] = carry;
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t v = lane < kRowsPerItem ? ftot[2 + lane] : 0u;
        const uint32_t inc = wave_inclusive_scan(v);
        if (lane < kRowsPerItem)
            cbase[lane] = ftot[1] + inc - v;
        if (lane == kWave - 1) {
            *tile_start_end = ftot[0];
            meta[kMetaItems] = ftot[1] + inc;
            meta[kMetaCursor] = 0u;
            meta[kMetaKeys] = (uint64_t)meta[kMetaRuns] * kKeyRunLength <= (uint64_t)meta[kMetaBinned] ? 1u : 0u;
        }
    }
    __syncthreads();
    for (int64_t i = threadIdx.x; i < nblocks * kRowsPerItem; i += 1024) {
        const int64_t k = i / kRowsPerItem;
        const int r = (int)(i % kRowsPerItem);
        part[k * kPlanStride + 2 + r] += cbase[r];
    }
}

template <int DIM>
__global__ void __launch_bounds__(kPlanBlock) plan_final_kernel(const uint32_t *__restrict__ tile_count,
                                                                int64_t n_tiles, const uint32_t *__restrict__ part,
                                                                const uint32_t *__restrict__ meta,
                                                                uint32_t *__restrict__ tile_start,
                                                                uint4 *__restrict__ items)
{
    constexpr uint32_t S = slice_records<DIM>();
    __shared__ uint32_t cls_next[kRowsPerItem];
    __shared__ uint32_t tot;
    const uint32_t *in = part + (int64_t)blockIdx.x * kPlanStride;
    if (threadIdx.x < kRowsPerItem)
        cls_next[threadIdx.x] = in[2 + threadIdx.x];
    const int64_t base = (int64_t)blockIdx.x * kPlanTiles + (int64_t)threadIdx.x * kPlanPer;
    uint32_t c[kPlanPer];
    uint32_t sc = 0, sf = 0;
#pragma unroll
    for (int i = 0; i < kPlanPer; ++i) {
        const int64_t t = base + i;
        c[i] = t < n_tiles ? tile_count[t] : 0u;
        uint32_t full, cls;
        tile_slices<DIM>(c[i], full, cls);
        sc += c[i];
        sf += full;
    }
    uint32_t rec0 = in[0] + block_exclusive_scan<kPlanBlock>(sc, &tot);
    uint32_t item0 = in[1] + block_exclusive_scan<kPlanBlock>(sf, &tot);
    __syncthreads();                                 // cls_next visible
    const uint32_t total = meta[0];
    auto place = [&](uint32_t q) { return q < (total + 1) / 2 ? 2 * q : 2 * (total - 1 - q) + 1; };
#pragma unroll
    for (int i = 0; i < kPlanPer; ++i) {
        const int64_t t = base + i;
        if (t >= n_tiles)
            break;
        tile_start[t] = rec0;
        uint32_t full, cls;
        tile_slices<DIM>(c[i], full, cls);
        for (uint32_t k = 0; k < full; ++k)
            items[place(item0 + k)] = make_uint4((uint32_t)t, rec0 + k * S, S, 0u);
        if (cls < (uint32_t)kRowsPerItem)
            items[place(atomicAdd(&cls_next[cls], 1u))] = make_uint4((uint32_t)t, rec0 + full * S, c[i] - full * S, 0u);
        item0 += full;
        rec0 += c[i];
    }
}

// Pass 5: each binned particle's record at its tile's first record plus its
// rank.  Particles outside the declared ranges are counted and written with
// zero mass, velocity and affine matrix: they contribute nothing, as if
// skipped.  Each thread loads two particles before writing either, so that
// twice the loads are in flight.  Every lane of a wavefront runs the same
// number of iterations, so all of them reach write_records's exchanges.  The
// streams read or written once (particle fields, ranks, slots, records) carry
// the nontemporal hint, which leaves the L2 to the one-byte cell keys: those
// land scattered and are merged into whole lines there (measured: 0.80 ->
// 0.75 ms for the 16M-particle blob binning; the keys themselves with the hint
// take 1.2 ms).
template <int DIM>
__device__ __forceinline__ void load_record(const Fields &f, int64_t p, float *rec)
{
    constexpr int R = rec_floats<DIM>();
    int fi = 0;
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        rec[fi++] = __builtin_nontemporal_load(&f.x[e * f.n + p]);
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        rec[fi++] = __builtin_nontemporal_load(&f.v[e * f.n + p]);
#pragma unroll
    for (int q = 0; q < DIM * DIM; ++q)
        rec[fi++] = f.C ? __builtin_nontemporal_load(&f.C[q * f.n + p]) : 0.0f;
    rec[fi++] = __builtin_nontemporal_load(&f.m[p]);
#pragma unroll
    for (; fi < R; ++fi)
        rec[fi] = 0.0f;
}

// Range check and destination of one loaded record: its index in the binned
// copy, or kEmpty when the particle is not binned.  KEEP: no range check (the
// record is copied as it is; the fused substep checks the ranges itself).
template <int DIM, bool KEEP>
__device__ __forceinline__ uint32_t place_record(const Fields &f, RangesF r, float nf, float dx, float last_base,
                                                 int ntx, int64_t p, float *rec,
                                                 const uint32_t *__restrict__ rank_in,
                                                 const uint32_t *__restrict__ tile_start,
                                                 uint32_t *__restrict__ slot_out, uint8_t *__restrict__ cell_key,
                                                 bool write_key, uint32_t *__restrict__ status)
{
    constexpr int R = rec_floats<DIM>();
    uint32_t t, l;
    if (!particle_cell<DIM>(rec, nf, dx, last_base, ntx, t, l)) {
        slot_out[p] = kEmpty;
        return kEmpty;
    }
    if constexpr (!KEEP) {
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
    }
    const uint32_t pos = tile_start[t] + __builtin_nontemporal_load(&rank_in[p]);
    __builtin_nontemporal_store(pos, &slot_out[p]);
    if (write_key)
        cell_key[pos] = (uint8_t)l;
    return pos;
}

typedef float v4nt __attribute__((ext_vector_type(4)));

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
                __builtin_nontemporal_store(v4nt{ v.x, v.y, v.z, v.w }, reinterpret_cast<v4nt *>(sorted + (int64_t)d * R) + piece);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        (void)stage;
        (void)spos;
        if (pos != kEmpty) {
            v4nt *dst = reinterpret_cast<v4nt *>(sorted + (int64_t)pos * R);
#pragma unroll
            for (int q = 0; q < R / 4; ++q)
                __builtin_nontemporal_store(v4nt{ rec[4 * q], rec[4 * q + 1], rec[4 * q + 2], rec[4 * q + 3] }, dst + q);
        }
    }
}

template <int DIM, bool KEEP>
__global__ void __launch_bounds__(kBinThreads) bin_scatter_kernel(Fields f, RangesF r, float nf, float dx,
                                                                   float last_base, int ntx, int64_t chunks, int per,
                                                                   const uint32_t *__restrict__ rank_in,
                                                                   const uint32_t *__restrict__ tile_start,
                                                                   uint32_t *__restrict__ slot_out,
                                                                   uint8_t *__restrict__ cell_key,
                                                                   const uint32_t *__restrict__ meta,
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
    const bool write_keys = !KEEP && meta[kMetaKeys] != 0u;
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
                da = place_record<DIM, KEEP>(f, r, nf, dx, last_base, ntx, pa, ra, rank_in, tile_start, slot_out,
                                             cell_key, write_keys, status);
            if (lb)
                db = place_record<DIM, KEEP>(f, r, nf, dx, last_base, ntx, pb, rb, rank_in, tile_start, slot_out,
                                             cell_key, write_keys, status);
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

hipError_t launch_bin(int dim, int n, const Fields &p, RangesF r, const BinView &b, uint32_t *status, hipStream_t s,
                      bool keep)
{
    const float nf = (float)n, dx = 1.0f / (float)n, last = (float)(n - 3);
    const int ntx = n / kTile;
    hipLaunchKernelGGL(bin_reset_kernel, dim3(blocks_for(b.n_tiles + kMetaWords, 256)), dim3(256), 0, s, b.tile_count,
                       b.n_tiles, b.meta, b.stamp);
    // particles per thread of a chunk: the smallest power of two from 4 to
    // kMaxPer that gives no more chunks than CUs (or kMaxPer)
    const int64_t span = (int64_t)kBinThreads * device_cu_count();
    int per = 4;
    while (per < kMaxPer && (int64_t)per * span < p.n)
        per *= 2;
    const int64_t chunks = (p.n + kBinThreads * per - 1) / (kBinThreads * per);
    const unsigned cblocks = (unsigned)(chunks < (int64_t)device_cu_count() ? chunks : device_cu_count());
    auto count = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(cblocks), dim3(kBinThreads), 0, s, p, nf, dx, last, ntx, chunks, b.tile_count,
                           b.rank, status, b.meta);
    };
    if (chunks > 0) {
        if (dim == 3) {
            switch (per) {
            case 4: count(bin_tile_count_kernel<3, 4>); break;
            case 8: count(bin_tile_count_kernel<3, 8>); break;
            case 16: count(bin_tile_count_kernel<3, 16>); break;
            case 32: count(bin_tile_count_kernel<3, 32>); break;
            default: count(bin_tile_count_kernel<3, kMaxPer>); break;
            }
        } else {
            switch (per) {
            case 4: count(bin_tile_count_kernel<2, 4>); break;
            case 8: count(bin_tile_count_kernel<2, 8>); break;
            case 16: count(bin_tile_count_kernel<2, 16>); break;
            case 32: count(bin_tile_count_kernel<2, 32>); break;
            default: count(bin_tile_count_kernel<2, kMaxPer>); break;
            }
        }
    }
    const int64_t pblocks = (b.n_tiles + kPlanTiles - 1) / kPlanTiles;
    uint4 *items = reinterpret_cast<uint4 *>(b.items);
    if (dim == 3) {
        hipLaunchKernelGGL(plan_reduce_kernel<3>, dim3((unsigned)pblocks), dim3(kPlanBlock), 0, s, b.tile_count,
                           b.n_tiles, b.scan_tmp);
        hipLaunchKernelGGL(plan_partials_kernel, dim3(1), dim3(1024), 0, s, b.scan_tmp, pblocks,
                           b.tile_start + b.n_tiles, b.meta);
        hipLaunchKernelGGL(plan_final_kernel<3>, dim3((unsigned)pblocks), dim3(kPlanBlock), 0, s, b.tile_count,
                           b.n_tiles, b.scan_tmp, b.meta, b.tile_start, items);
    } else {
        hipLaunchKernelGGL(plan_reduce_kernel<2>, dim3((unsigned)pblocks), dim3(kPlanBlock), 0, s, b.tile_count,
                           b.n_tiles, b.scan_tmp);
        hipLaunchKernelGGL(plan_partials_kernel, dim3(1), dim3(1024), 0, s, b.scan_tmp, pblocks,
                           b.tile_start + b.n_tiles, b.meta);
        hipLaunchKernelGGL(plan_final_kernel<2>, dim3((unsigned)pblocks), dim3(kPlanBlock), 0, s, b.tile_count,
                           b.n_tiles, b.scan_tmp, b.meta, b.tile_start, items);
    }
    // the scatter's own blocks: two or more per CU
    const int64_t sspan = (int64_t)kBinThreads * device_cu_count() * 2;
    int64_t sper = (p.n + sspan - 1) / sspan;
    sper = sper < 4 ? 4 : (sper > kScatterPer ? kScatterPer : sper);
    const int64_t schunks = (p.n + kBinThreads * sper - 1) / (kBinThreads * sper);
    const unsigned sblocks = (unsigned)(schunks < (int64_t)device_cu_count() * 8 ? schunks : device_cu_count() * 8);
    auto scatter = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(sblocks), dim3(kBinThreads), 0, s, p, r, nf, dx, last, ntx, schunks, (int)sper,
                           b.rank, b.tile_start, b.slot, b.cell_key, b.meta, b.sorted, status);
    };
    if (chunks > 0) {
        if (dim == 3)
            keep ? scatter(bin_scatter_kernel<3, true>) : scatter(bin_scatter_kernel<3, false>);
        else
            keep ? scatter(bin_scatter_kernel<2, true>) : scatter(bin_scatter_kernel<2, false>);
    }
    return hipGetLastError();
}

namespace {

// Copies each binned particle's x, v and C from its record back to the
// caller's component-major arrays (m is never changed by a substep).
template <int DIM>
__global__ void __launch_bounds__(256) gather_records_kernel(int64_t np, const uint32_t *__restrict__ slot,
                                                             const float *__restrict__ sorted, float *__restrict__ x,
                                                             float *__restrict__ v, float *__restrict__ C,
                                                             const uint32_t *__restrict__ meta, BinStamp stamp,
                                                             uint32_t *__restrict__ status)
{
    constexpr int R = rec_floats<DIM>();
    if (!stamp_matches(meta, stamp, false)) {        // binned for another grid or count: copy nothing
        if (blockIdx.x == 0 && threadIdx.x == 0)
            atomicAdd(&status[3], 1u);
        return;
    }
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t r = slot[p];
        if (r == kEmpty)
            continue;
        const float4 *src = reinterpret_cast<const float4 *>(sorted + (int64_t)r * R);
        float rec[R];
#pragma unroll
        for (int q = 0; q < R / 4; ++q) {
            const float4 t = src[q];
            rec[4 * q] = t.x;
            rec[4 * q + 1] = t.y;
            rec[4 * q + 2] = t.z;
            rec[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int d = 0; d < DIM; ++d) {
            x[d * np + p] = rec[d];
            v[d * np + p] = rec[DIM + d];
        }
#pragma unroll
        for (int q = 0; q < DIM * DIM; ++q)
            C[q * np + p] = rec[2 * DIM + q];
    }
}

}  // namespace

hipError_t launch_gather_records(int dim, int64_t np, const BinView &b, float *x, float *v, float *C,
                                 uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    if (dim == 3)
        hipLaunchKernelGGL(gather_records_kernel<3>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, b.slot, b.sorted,
                           x, v, C, b.meta, b.stamp, status);
    else
        hipLaunchKernelGGL(gather_records_kernel<2>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, b.slot, b.sorted,
                           x, v, C, b.meta, b.stamp, status);
    return hipGetLastError();
}

}  // namespace mpmk
