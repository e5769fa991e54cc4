// p2g_device.hpp -- device code shared by the P2G kernels (p2g.hip) and the
// fused substep kernel (fused.hip).
//
// The transfer ("Implementation -- GPU Optimization & Reference Codebases",
// sections 1, 2.1 and 3.1): every particle deposits mass m w and APIC momentum
// m w (v + C (x_i - x_p)) on the 3^dim nodes of its quadratic B-spline
// stencil; each contribution is scaled by S = 2^k and rounded to an integer
// once, so node sums are integer sums and the grid does not depend on the
// order in which particles arrive.
//
// Fixed operation order per particle and node (a, b, c), float32:
//   wmS = (((m*S) * wx[a]) * wy[b]) * wz[c]
//   u_d = ((v_d + C_d0*rx[a]) + C_d1*ry[b]) + C_d2*rz[c]
//   M += rint(wmS);  P_d += rint(wmS * u_d)
// The kernels hoist the per-(a), per-(a,b) and per-(c) partial products; the
// hoisted values are the same operations on the same operands, so every
// contribution has the same bits as the per-node form.

#pragma once

#include "common.hpp"

namespace mpmk {
namespace {

template <int DIM>
struct Particle {
    float x[DIM], v[DIM], C[DIM * DIM], m;
};

template <int DIM>
__device__ __forceinline__ bool in_ranges(const Particle<DIM> &p, RangesF r)
{
    bool ok = fabsf(p.m) <= r.max_mass;
#pragma unroll
    for (int d = 0; d < DIM; ++d)
        ok = ok && (fabsf(p.v[d]) <= r.max_speed);
#pragma unroll
    for (int k = 0; k < DIM * DIM; ++k)
        ok = ok && (fabsf(p.C[k]) <= r.max_affine);
    return ok;
}

// Per-particle factors shared by the stencil's nodes.
template <int DIM>
struct Hoisted {
    float mwxy[3][3];          // ((m*S)*wx[a])*wy[b]
    float t2[DIM][3][3];       // (v_d + C_d0*rx[a]) + C_d1*ry[b]
    float wz[3];
    float cz[DIM][3];          // C_d2*rz[c]
    int base[DIM];
};

template <int DIM>
__device__ __forceinline__ bool hoist(const Particle<DIM> &p, float nf, float dx, float last_base, float S,
                                      Hoisted<DIM> &h)
{
    Axis ax[DIM];
    bool ok = true;
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        ok = axis_stencil(p.x[e], nf, dx, last_base, ax[e]) && ok;
        h.base[e] = ax[e].base;
    }
    const float mS = p.m * S;
    const float wx[3] = { ax[0].w0, ax[0].w1, ax[0].w2 };
    const float wy[3] = { ax[1].w0, ax[1].w1, ax[1].w2 };
    const float rx[3] = { ax[0].r0, ax[0].r1, ax[0].r2 };
    const float ry[3] = { ax[1].r0, ax[1].r1, ax[1].r2 };
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const float mwx = mS * wx[a];
#pragma unroll
        for (int b = 0; b < 3; ++b)
            h.mwxy[a][b] = mwx * wy[b];
    }
#pragma unroll
    for (int d = 0; d < DIM; ++d) {
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const float t1 = p.v[d] + p.C[d * DIM + 0] * rx[a];
#pragma unroll
            for (int b = 0; b < 3; ++b)
                h.t2[d][a][b] = t1 + p.C[d * DIM + 1] * ry[b];
        }
    }
    if constexpr (DIM == 3) {
        const float rz[3] = { ax[2].r0, ax[2].r1, ax[2].r2 };
        h.wz[0] = ax[2].w0;
        h.wz[1] = ax[2].w1;
        h.wz[2] = ax[2].w2;
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int c = 0; c < 3; ++c)
                h.cz[d][c] = p.C[d * DIM + 2] * rz[c];
    }
    return ok;
}

template <int DIM>
__device__ __forceinline__ void load_particle(const Fields &f, int64_t i, Particle<DIM> &p)
{
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        p.x[e] = f.x[e * f.n + i];
        p.v[e] = f.v[e * f.n + i];
    }
#pragma unroll
    for (int k = 0; k < DIM * DIM; ++k)
        p.C[k] = f.C ? f.C[k * f.n + i] : 0.0f;
    p.m = f.m[i];
}

__device__ __forceinline__ void atomic_add_i64(int64_t *addr, int64_t v)
{
    atomicAdd(reinterpret_cast<unsigned long long *>(addr), (unsigned long long)v);
}

// Every contribution of one hoisted particle to the grid, one 64-bit global
// atomic each.
template <int DIM>
__device__ __forceinline__ void deposit_direct(const Hoisted<DIM> &h, int n, int64_t nodes, int64_t *__restrict__ grid)
{
    const int nc = DIM == 3 ? 3 : 1;
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int c = 0; c < nc; ++c) {
                float wmS = h.mwxy[a][b];
                int64_t node;
                if constexpr (DIM == 3) {
                    wmS = wmS * h.wz[c];
                    node = ((int64_t)(h.base[2] + c) * n + (h.base[1] + b)) * n + (h.base[0] + a);
                } else {
                    node = (int64_t)(h.base[1] + b) * n + (h.base[0] + a);
                }
                atomic_add_i64(&grid[node], (int64_t)rintf(wmS));
#pragma unroll
                for (int d = 0; d < DIM; ++d) {
                    float u = h.t2[d][a][b];
                    if constexpr (DIM == 3)
                        u = u + h.cz[d][c];
                    atomic_add_i64(&grid[(1 + d) * nodes + node], (int64_t)rintf(wmS * u));
                }
            }
}

// ---------------------------------------------------------------------------
template <int DIM>
__global__ void __launch_bounds__(256) p2g_direct_kernel(Fields f, const uint32_t *__restrict__ order, int n,
                                                          float nf, float dx, float last_base, float S, RangesF r,
                                                          int64_t *__restrict__ grid, uint32_t *__restrict__ status)
{
    const int64_t nodes = DIM == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < f.n;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = order ? (int64_t)order[k] : k;
        if (i >= f.n) {                  // an order entry that names no particle
            atomicAdd(&status[3], 1u);
            continue;
        }
        Particle<DIM> p;
        load_particle<DIM>(f, i, p);
        Hoisted<DIM> h;
        const bool dom = hoist<DIM>(p, nf, dx, last_base, S, h);
        const bool rng = dom && in_ranges<DIM>(p, r);
        wave_count(!dom, &status[0]);
        wave_count(dom && !rng, &status[1]);
        if (!rng)
            continue;
        deposit_direct<DIM>(h, n, nodes, grid);
    }
}

// ---------------------------------------------------------------------------
// Tiled path.  The bins hold each tile's particle records (64 bytes: x, v, C,
// m in 3D) in one contiguous range with each record's cell key beside it, cut
// into slices of at most slice_records(), one work item each.  A wavefront
// takes one item and first sorts the slice by cell in LDS into rows of group
// entries: each cell completed to whole groups of kGroup entries (a
// completing entry names one of the cell's records, read with zero mass), and
// the groups laid out "transposed": group g of an item with R rows sits in
// lane g / R of row g % R.  Every lane then holds kGroup particles of one
// cell, and the 64 lanes are R groups apart in cell order, so they are mostly
// in different cells and write different node addresses at the same
// instruction.  The records a row names lie in the slice's contiguous range.
//
// Per lane and stencil node, the group's kGroup quantised contributions are
// summed in float64 registers and added to the on-chip node block with one LDS
// atomic, a quarter of the atomics of one add per particle (the implementation
// page's section 2.1 pre-reduces same-node contributions before one atomic).
//
// The tile's node block ((4+2)^dim nodes, 1+dim channels) lives in LDS as
// float64.  Every contribution is an integer below 2^53 in magnitude and the
// bounds check keeps every partial sum of one work item below 2^53, so each
// add is exact and the block holds the exact integer sums in any order.  After
// the item the block is flushed with one 64-bit global atomic per non-zero
// node and channel ("Implementation -- GPU Optimization & Reference
// Codebases", section 2.1: stage a tile of the grid on chip, accumulate there,
// flush once).
// ---------------------------------------------------------------------------
template <int DIM>
struct TileShape {
    static constexpr int side = kTile + 2;
    static constexpr int nodes = DIM == 3 ? side * side * side : side * side;
    static constexpr int cells = DIM == 3 ? kTile * kTile * kTile : kTile * kTile;
    static constexpr int ch = 1 + DIM;
};

// Per-particle factors of the grouped kernel (the per-(a,b) products are
// formed inside the node loop to keep kGroup particles' state in registers).
template <int DIM>
struct GroupHoist {
    float mwx[3];              // (m*S)*wx[a]
    float wy[3];
    float wz[3];
    float t1[DIM][3];          // v_d + C_d0*rx[a]
    float cy[DIM][3];          // C_d1*ry[b]
    float cz[DIM][3];          // C_d2*rz[c]
    int base[DIM];
};

template <int DIM>
__device__ __forceinline__ void group_hoist(const float *rec, float nf, float dx, float last_base, float S,
                                            GroupHoist<DIM> &h)
{
    Axis ax[DIM];
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        axis_stencil(rec[e], nf, dx, last_base, ax[e]);
        h.base[e] = ax[e].base;
    }
    const float *v = rec + DIM, *C = rec + 2 * DIM, m = rec[2 * DIM + DIM * DIM];
    const float mS = m * S;
    const float wx[3] = { ax[0].w0, ax[0].w1, ax[0].w2 }, rx[3] = { ax[0].r0, ax[0].r1, ax[0].r2 };
    const float ry[3] = { ax[1].r0, ax[1].r1, ax[1].r2 };
    h.wy[0] = ax[1].w0;
    h.wy[1] = ax[1].w1;
    h.wy[2] = ax[1].w2;
#pragma unroll
    for (int a = 0; a < 3; ++a)
        h.mwx[a] = mS * wx[a];
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int o = 0; o < 3; ++o) {
            h.t1[d][o] = v[d] + C[d * DIM + 0] * rx[o];
            h.cy[d][o] = C[d * DIM + 1] * ry[o];
        }
    if constexpr (DIM == 3) {
        const float rz[3] = { ax[2].r0, ax[2].r1, ax[2].r2 };
        h.wz[0] = ax[2].w0;
        h.wz[1] = ax[2].w1;
        h.wz[2] = ax[2].w2;
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int o = 0; o < 3; ++o)
                h.cz[d][o] = C[d * DIM + 2] * rz[o];
    }
}

struct TiledArgs {
    const float *sorted;
    const uint8_t *cell_key;               // the records' cell keys, when the binning wrote them
    const uint32_t *items, *meta;
    uint32_t *cursor;
    int n, ntx;
    float nf, dx, last_base, S;
    int64_t *grid;
    uint32_t *status;
    BinStamp stamp;                        // the binning these bins must come from
};

__global__ void reset_cursor_kernel(uint32_t *cursor) { *cursor = 0u; }

// Group entries of the item being processed, in LDS: a record's offset in the
// slice, with kPad16 set when the entry only completes its cell's last group
// (read with zero mass).  Group P of an item sits in lane P % 64 of row P / 64,
// its kGroup entries at ent[kGroup * P ...].
constexpr uint16_t kPad16 = 0x8000u;
constexpr int kKeyWords = 8;                  // words of four cell keys per lane: a whole slice
constexpr uint32_t kMaxGroups = kRowsPerItem * kWave;
constexpr uint32_t kTrashEntry = kMaxGroups * kGroup;      // spare group entry

// Counting sort of the item's records by cell into groups ("Particle worlds,
// part 3", steps 3-4, on chip).  The slice's cell keys are read once, four to
// a word, and kept in registers.  One returning LDS atomic per key on its
// cell's counter gives both the histogram and the key's rank among its cell's
// keys, and every key also leaves its record's offset in its cell's
// representative slot (any one of them survives).  Cell c holds
// g_c = ceil(n_c / kGroup) groups; group k of cell c (records kGroup k ..
// kGroup k + kGroup - 1 by rank, the last one completed with pad entries that
// name the representative record) is placed level by level: all cells' groups
// 0 in cell order, then all groups 1, and so on, so that the 64 lanes of a row
// hold groups of 64 different cells wherever the level is wide enough (they
// then add to different LDS nodes, and with cells numbered x, z, y a full
// level's lanes hit distinct banks).  gpos[cg_c + k] is that place, cg_c the
// cell's first group in cell order.  Positions past the slice's keys in a word
// that holds some take their atomics and representative writes on a spare
// slot of their own lane (kWave + lane) and their entry writes on a spare
// entry, so that inside each round of words the code has no branches and the
// LDS operations of many keys are in flight at once.  One wavefront.  The
// keys are read by load_keys: the cell key of record `first` + i is byte i of
// the key array, whose allocation extends to a multiple of 4 bytes past the
// last key.  Returns the number of groups (at most kMaxGroups for a slice of
// at most slice_records()).
__device__ __forceinline__ void load_keys(const uint8_t *__restrict__ keys, uint32_t first, uint32_t count, int lane,
                                          uint32_t kw[kKeyWords])
{
    const uint32_t off = first & 3u;
    const uint32_t *words = reinterpret_cast<const uint32_t *>(keys + (first - off));
    const uint32_t n_words = (off + count + 3u) / 4u;
    const uint32_t last_word = n_words - 1u;
    const int rounds = (int)((n_words + kWave - 1) / kWave);
#pragma unroll
    for (int k = 0; k < kKeyWords; ++k) {
        const uint32_t i = (uint32_t)(k * kWave + lane);
        kw[k] = k < rounds ? words[i < last_word ? i : last_word] : 0u;
    }
}

// The same packing of keys computed from the records themselves: the key of
// slice position s is the local number (tile_local) of the base cell of
// record first + s inside the tile whose first cell is torg, with
// base = floor(x n - 1/2) per axis exactly as the binning computes it.  Each
// axis offset is masked to the tile, so a key is below kWave even for a record
// outside its tile (never in correct use; the rows check such a group and
// count it in status[3]).  Records are read by their first 16 bytes (x).
template <int DIM>
__device__ __forceinline__ void record_keys(const float *__restrict__ sorted, uint32_t first, uint32_t count,
                                            const int (&torg)[3], float nf, int lane, uint32_t kw[kKeyWords])
{
    constexpr int R = rec_floats<DIM>();
    const uint32_t off = first & 3u;
    const uint32_t n_words = (off + count + 3u) / 4u;
    const int rounds = (int)((n_words + kWave - 1) / kWave);
#pragma unroll
    for (int k = 0; k < kKeyWords; ++k) {
        kw[k] = 0u;
        if (k >= rounds)
            continue;
        float4 xs[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t s = 4u * (uint32_t)(k * kWave + lane) + (uint32_t)b - off;
            xs[b] = s < count ? *reinterpret_cast<const float4 *>(sorted + (int64_t)(first + s) * R)
                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float xe[3] = { xs[b].x, xs[b].y, xs[b].z };
            uint32_t l[DIM];
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                l[e] = (uint32_t)((int)floorf(xe[e] * nf - 0.5f) - torg[e]) & (uint32_t)(kTile - 1);
            kw[k] |= tile_local<DIM>(l) << (8 * b);
        }
    }
}

// `kw` holds the slice's keys as load_keys or record_keys left them; cnt must be zero on
// entry (all 2 kWave slots), and the call leaves it so for the next item.
// STRAYS: a key of kWave or more marks a record outside the tile, which gets
// no group (its entry goes to the spare entry).
template <bool STRAYS>
__device__ __forceinline__ uint32_t sort_item(const uint32_t kw[kKeyWords], uint32_t first, uint32_t count,
                                              uint16_t *ent, uint16_t *gpos, uint32_t *cnt, uint32_t *cgs,
                                              uint32_t *rep, int lane)
{
    const uint32_t off = first & 3u;
    const uint32_t n_words = (off + count + 3u) / 4u;
    const int rounds = (int)((n_words + kWave - 1) / kWave);   // rounds of one word per lane
    // rank of key (k, b) among its cell's keys (spare slots: meaningless); the
    // results are only read after the barrier, so the atomics queue up
    uint32_t rk[kKeyWords][4];
#pragma unroll
    for (int k = 0; k < kKeyWords; ++k) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            rk[k][b] = 0u;
        if (k >= rounds)
            continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t s = 4u * (uint32_t)(k * kWave + lane) + (uint32_t)b - off;
            const uint32_t byte = (kw[k] >> (8 * b)) & 0xFFu;
            const bool live = s < count && (!STRAYS || byte < (uint32_t)kWave);
            const uint32_t key = live ? byte : kWave + (uint32_t)lane;
            rk[k][b] = atomicAdd(&cnt[key], 1u);
            rep[key] = s;
        }
    }
    __syncthreads();
    const uint32_t n_l = cnt[lane];
    const uint32_t g_l = (n_l + kGroup - 1) / kGroup;
    cnt[lane] = 0u;                                            // ready for the next item
    cnt[kWave + lane] = 0u;
    const uint32_t inc = wave_inclusive_scan(g_l);
    const uint32_t groups = (uint32_t)__shfl((int)inc, kWave - 1, kWave);
    const uint32_t cg = inc - g_l;
    cgs[lane] = cg;
    // level by level: this lane's cell takes the next free places of every
    // level it reaches, in cell order among that level's cells
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t level_start = 0;
    for (uint32_t k = 0;; ++k) {
        const bool active = g_l > k;
        const uint64_t m = __ballot(active);
        if (m == 0ull)
            break;
        if (active)
            gpos[cg + k] = (uint16_t)(level_start + (uint32_t)__popcll(m & below));
        level_start += (uint32_t)__popcll(m);
    }
    // this lane's cell's pads complete its last group
    for (uint32_t q = n_l; q < kGroup * g_l; ++q)
        ent[kGroup * (uint32_t)gpos[cg + q / kGroup] + q % kGroup] = (uint16_t)(kPad16 | rep[lane]);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKeyWords; ++k) {
        if (k >= rounds)
            continue;
        uint32_t g4[4];
        bool live[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t s = 4u * (uint32_t)(k * kWave + lane) + (uint32_t)b - off;
            const uint32_t byte = (kw[k] >> (8 * b)) & 0xFFu;
            live[b] = s < count && (!STRAYS || byte < (uint32_t)kWave);
            g4[b] = live[b] ? cgs[byte] + rk[k][b] / kGroup : 0u;
        }
        uint32_t p4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            p4[b] = gpos[g4[b]];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t s = 4u * (uint32_t)(k * kWave + lane) + (uint32_t)b - off;
            const uint32_t e = kGroup * p4[b] + rk[k][b] % kGroup;
            ent[live[b] ? e : kTrashEntry] = (uint16_t)s;
        }
    }
    __syncthreads();
    return groups;
}

// Range check of one binned record (x, v, C, m): the declared ranges as at
// binning.
template <int DIM>
__device__ __forceinline__ bool record_in_ranges(const float *rec, RangesF r)
{
    bool ok = fabsf(rec[2 * DIM + DIM * DIM]) <= r.max_mass;
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        ok = ok && fabsf(rec[DIM + e]) <= r.max_speed;
#pragma unroll
    for (int q = 0; q < DIM * DIM; ++q)
        ok = ok && fabsf(rec[2 * DIM + q]) <= r.max_affine;
    return ok;
}

// The rows of one work item: per lane and row, the group's kGroup records
// (entries ent, offsets from `first`), their quantised contributions summed
// per node and channel in float64 registers and added to the node block acc
// with one LDS atomic.  CHECK: records are range-checked here (out-of-range
// records add nothing and are counted in status[1]).
template <int DIM, bool CHECK>
__device__ __forceinline__ void item_rows(const TiledArgs &a, RangesF r, uint32_t first, uint32_t rows,
                                          uint32_t groups, const uint16_t *ent, double *acc, const int (&torg)[3],
                                          int lane)
{
    using TS = TileShape<DIM>;
    constexpr int R = rec_floats<DIM>();
    constexpr int G = kGroup;
    uint32_t bad = 0;
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
            const bool pad = (e4[k] & kPad16) != 0;
            if constexpr (CHECK) {
                // the declared ranges, checked here instead of at binning:
                // a record outside them adds nothing and is counted once
                if (!pad && !record_in_ranges<DIM>(rec, r)) {
                    ++bad;
#pragma unroll
                    for (int q = DIM; q < R; ++q)
                        rec[q] = 0.0f;
                }
            }
            // a pad completes the cell's group and adds nothing: its record (one
            // of the cell's, for the cell's position) is read with zero mass,
            // velocity and affine matrix, so its products are exact zeros even
            // where that record holds values outside the ranges (Inf, NaN)
            if (pad) {
#pragma unroll
                for (int q = DIM; q < R; ++q)
                    rec[q] = 0.0f;
            }
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
    if constexpr (CHECK) {
        if (bad != 0u)
            atomicAdd(&a.status[1], bad);
    }
}

}  // namespace
}  // namespace mpmk
