// p2g.hip -- particle-to-grid scatter kernels for gfx950.
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
// Direct path: one thread per particle, 64-bit global atomics per
// contribution.  No binning needed; the baseline the tiled path is measured
// against and the path for unbinned particle sets.
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
    const uint8_t *cell_key;
    const uint32_t *items, *meta;
    uint32_t *cursor;
    int n, ntx;
    float nf, dx, last_base, S;
    int64_t *grid;
    uint32_t *status;
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

// `kw` holds the slice's keys as load_keys left them; cnt must be zero on
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
            if (pad)                                     // completes the cell's group: zero mass
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
    if constexpr (CHECK) {
        if (bad != 0u)
            atomicAdd(&a.status[1], bad);
    }
}

template <int DIM>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
p2g_tiled_kernel(TiledArgs a)
{
    using TS = TileShape<DIM>;
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
    const uint32_t n_items = a.meta[0];
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
    // during the current item's flush, so no round trip stalls the wave
    // between items.
    const uint4 *items = reinterpret_cast<const uint4 *>(a.items);
    uint32_t next = 0;
    if (lane == 0)
        next = atomicAdd(a.cursor, 1u);
    uint32_t item = __builtin_amdgcn_readfirstlane(next);
    uint4 rec_item = make_uint4(0u, 0u, 0u, 0u);
    uint32_t kw[kKeyWords];
    if (item < n_items) {
        rec_item = items[item];
        load_keys(a.cell_key, rec_item.y, rec_item.z, lane, kw);
    }
    for (;;) {
        if (item >= n_items)
            break;
        if (lane == 0)
            next = atomicAdd(a.cursor, 1u);
        // item: tile, first record, records (one slice of the tile)
        const uint32_t tile = rec_item.x, first = rec_item.y, count = rec_item.z;
        int torg[3] = { 0, 0, 0 };
        {
            uint32_t t = tile;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                torg[e] = (int)(t % (uint32_t)a.ntx) * kTile;
                t /= (uint32_t)a.ntx;
            }
        }
        const uint32_t groups = sort_item<false>(kw, first, count, ent, gpos, cnt, cgs, rep, lane);
        const uint32_t rows = (groups + kWave - 1) / kWave;
        const uint32_t item_next = __builtin_amdgcn_readfirstlane(next);
        uint4 rec_next = make_uint4(0u, 0u, 0u, 0u);
        if (item_next < n_items)
            rec_next = items[item_next];
        item_rows<DIM, false>(a, RangesF{ 0.0f, 0.0f, 0.0f }, first, rows, groups, ent, acc, torg, lane);
        __syncthreads();
        item = item_next;
        rec_item = rec_next;
        if (item < n_items)
            load_keys(a.cell_key, rec_item.y, rec_item.z, lane, kw);
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
// Fused grid-to-particle and particle-to-grid per work item ("Implementation
// -- GPU Optimization & Reference Codebases", section 2.1: one kernel per
// tile slice loads the tile's node block with its halo, applying the grid
// update as it loads, gathers and updates the slice's particles, and scatters
// them into the next grid through the on-chip block).  The particle state is
// the binned records, updated in place.  Per item:
//  1. the grid velocity of the (kTile+4)^dim nodes from one node below the
//     tile to six above (every node a particle of the tile can read after
//     drifting less than a cell) is formed from grid_in with node_velocity
//     into LDS (sharing the node block's memory);
//  2. each record is gathered and advected (g2p_particle, the same arithmetic
//     as the G2P kernel; a particle whose stencil leaves that window reads
//     grid_in directly) and written back; its cell in the new position is its
//     key, or a stray mark when it has left the tile;
//  3. the keys are sorted on chip as in the P2G kernel and the rows deposit
//     the updated records into the tile's node block (range checks here, not
//     at binning); strays deposit with global atomics;
//  4. the block is flushed to grid_out, and every node tile this item wrote
//     is flagged in tiles_out (for the restricted clear of that grid later).
// With grid_in NULL only steps 2 (keys), 3 and 4 run: the deposit of the
// records as they are.
// ---------------------------------------------------------------------------
struct FusedArgs {
    TiledArgs t;               // sorted: the records; grid: grid_out
    float *records;            // the same records, written
    const int64_t *grid_in;    // grid velocity source, or NULL for a deposit only
    uint8_t *tiles_out;        // node-tile flags of grid_out
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
    const uint32_t n_items = a.meta[0];
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
        // 2. gather and advect each record (with grid_in), then its key; the
        //    next record of the lane is loaded while this one is computed
        uint32_t clamps = 0;
        float4 nxt[R / 4];
        if ((uint32_t)lane < count) {
            const float4 *src = reinterpret_cast<const float4 *>(f.records + (int64_t)(first + lane) * R);
#pragma unroll
            for (int q = 0; q < R / 4; ++q)
                nxt[q] = src[q];
        }
        for (uint32_t i = (uint32_t)lane; i < count; i += kWave) {
            float4 *src = reinterpret_cast<float4 *>(f.records + (int64_t)(first + i) * R);
            float rec[R];
#pragma unroll
            for (int q = 0; q < R / 4; ++q) {
                rec[4 * q] = nxt[q].x;
                rec[4 * q + 1] = nxt[q].y;
                rec[4 * q + 2] = nxt[q].z;
                rec[4 * q + 3] = nxt[q].w;
            }
            if (i + kWave < count) {
                const float4 *ns = reinterpret_cast<const float4 *>(f.records + (int64_t)(first + i + kWave) * R);
#pragma unroll
                for (int q = 0; q < R / 4; ++q)
                    nxt[q] = ns[q];
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
    a.cursor = b.meta + 3;
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

hipError_t launch_g2p2g(int dim, int n, int frac_bits, const BinView &b, RangesF r, const int64_t *grid_in,
                        int64_t *grid_out, uint8_t *tiles_out, float dt, const float *gravity, int sticky,
                        uint32_t *status, hipStream_t s)
{
    FusedArgs f;
    TiledArgs &a = f.t;
    a.sorted = b.sorted;
    a.cell_key = b.cell_key;
    a.items = b.items;
    a.meta = b.meta;
    a.cursor = b.meta + 3;
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
