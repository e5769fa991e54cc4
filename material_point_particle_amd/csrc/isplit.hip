// isplit.hip -- integer-split quadratic APIC transfer.
//
// "particle to grid transfer in checked integer arithmetic", sections
// "integers do not care about order" and "what is not claimed": a quantity is
// split between the nodes of its stencil with the far shares rounded once and
// the near share taking the rest, so the shares sum to the quantity exactly
// and the node totals do not depend on the order particles arrive in.  The
// page names quadratic weights and the affine term as further splits of the
// same kind; this file carries that out.
//
// Positions are integers in 2^-16 cell.  With base = floor(x - 1/2) and
// F = x - base (in [2^15, 3 2^15), f = F / 2^16), the quadratic B-spline
// weights of the three nodes are
//   w_0 = (3 2^15 - F)^2 / 2^33,  w_2 = (F - 2^15)^2 / 2^33,  w_1 = 1 - w_0 - w_2,
// and the first moments u_o = w_o (o - f) are
//   u_0 = -(3 2^15 - F)^2 F / 2^49,  u_2 = (F - 2^15)^2 (2^17 - F) / 2^49,
//   u_1 = -u_0 - u_2,
// all exact dyadic rationals.  A quantity q is split along one axis into
// s_0 = round(q c_0), s_2 = round(q c_2) (the product formed exactly in 128
// bits, rounded to nearest with ties to even) and s_1 = q - s_0 - s_2 (for
// w) or -s_0 - s_2 (for u).  The 3^dim stencil shares are the split along x,
// each x share split along y, each of those along z.
//
// The transfer adds, at node i, m w_i (v + C (i - x)): channel 0 is the split
// of m; channel 1 + d is the split of m v_d plus, for every axis e, the split
// of m C_de with the first moments on axis e and the weights on the others.
//
// Two paths, both exact: integer additions commute, so the grid is
// bit-identical in every order, every launch and every path.
//  - direct: one thread per particle; its 3^dim shares of one channel are
//    formed in registers and added with one 64-bit global atomic each
//    (27 x 4 random atomics per particle in 3D);
//  - tiled: a counting sort of the particles into 8^dim-cell tiles, each
//    visited particle copied into a record in tile order (128 bytes; 64 in
//    the narrow path, whose quantities fit in 32 bits), then
//    one workgroup per slice of a tile accumulates the tile's 10^dim-node
//    block on chip with 64-bit LDS atomics and flushes it with one global
//    atomic per non-zero node and channel, consecutive lanes on consecutive
//    x nodes.
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace mpmk {
namespace {

struct AxisCoef {
    int64_t w0, w2;   // weights times 2^33
    int64_t u0, u2;   // first moments times 2^49
};

__device__ __forceinline__ AxisCoef axis_coef(int64_t F)
{
    const int64_t a = 3 * 32768 - F, b = F - 32768;
    AxisCoef c;
    c.w0 = a * a;
    c.w2 = b * b;
    c.u0 = -(a * a) * F;
    c.u2 = (b * b) * (131072 - F);
    return c;
}

// t / 2^K rounded to nearest, ties to even, for a 128-bit t whose quotient
// fits in 64 bits.
template <int K>
__device__ __forceinline__ int64_t round_shift(__int128 t)
{
    const int64_t fl = (int64_t)(t >> K);
    const uint64_t r = (uint64_t)t & ((1ull << K) - 1ull);
    const uint64_t half = 1ull << (K - 1);
    return fl + (int64_t)((r > half) | ((r == half) & ((uint64_t)fl & 1ull)));
}

// The narrow path (every split quantity below 2^28 in magnitude) forms each
// rounded product from 32 x 32 -> 64-bit multiply-adds, with the shares
// kept in 32 bits and biased so that they stay non-negative.  Every value
// entering a split along axis e carries the bias B_e = 3^(dim - e) b
// (b = 2^27 + 2^23 + 1, odd) and every share leaving it B_(e+1) (the last
// axis' shares b).  A share is at most 3/4 |q| + 1 in magnitude (a weight is
// at most 3/4, a first moment at most 1/4 in magnitude, and a near share adds
// the two roundings of the outer ones), so the values entering every axis'
// splits stay below 2^28 + 2 < 2 b in magnitude, and 27 b + 2^28 < 2^32:
// every biased value lies in [0, 2^32).  Because B_e = 3 B_(e+1), the near share of a
// weight split is q - s_0 - s_2 on the biased values as it is on the plain
// ones, and a first-moment split's is 3 B_(e+1) - s_0 - s_2.  A node's
// channel sum starts at minus the bias of the shares it will receive, so it
// ends at the plain sum (32-bit arithmetic modulo 2^32, whose result fits).
//
// A weight product (0 <= c <= 2^32) is one unsigned multiply-add: with
// q = q' - B_e, u = q' (c mod 2^32) + k with k = (1 + 2 B_(e+1)) 2^32 - B_e c
// is q c + 2^32 + 2 B_(e+1) 2^32 (half the divisor, then a shift of the high
// word) once q' is added to its high word where c = 2^32 (a weight of
// exactly one half, the only one whose low word is not c; such a weight
// exists only for a particle half a cell from a node, so that addition is
// made only in the wavefronts that hold one).  The high word is
// V' = V + 2 B_(e+1), V that of q c + 2^32: V / 2 rounds half up, and a tie
// (low word 0, V even) whose rounded-up quotient is odd (V = 2 mod 4, that
// is V' = 0 mod 4, B_(e+1) being odd) steps down by one.  The biased share
// (V' - tie) / 2 is formed as (V' - 1 + min(t, 1)) / 2 with
// t = (V' mod 4) | low word, zero exactly at such a tie.
constexpr uint32_t kShareBias = (1u << 27) + (1u << 23) + 1u;

template <int DIM, int E>
constexpr uint32_t axis_bias()
{
    uint32_t b = kShareBias;
    for (int i = E; i < DIM; ++i)
        b *= 3u;
    return b;
}

struct BiasedCoef {
    uint32_t c;       // the weight's low word
    uint32_t half;    // all ones for c = 2^32, else 0
    uint64_t k;
};

// A first moment (|c| < 2^49) as two signed 32-bit words: c = hi 2^32 + lo
// with lo in [-2^31, 2^31) (the low word read as signed, hi taking the rest).
struct NarrowCoef {
    int32_t hi, lo;
};

struct BiasedAxis {
    BiasedCoef w0, w2;
    NarrowCoef u0, u2;
};

template <int DIM, int E>
__device__ __forceinline__ BiasedCoef biased_coef(int64_t c)
{
    constexpr uint64_t bin = axis_bias<DIM, E>(), bout = axis_bias<DIM, E + 1>();
    const uint64_t k = ((1ull + 2ull * bout) << 32) - bin * (uint64_t)c;
    return BiasedCoef{ (uint32_t)(uint64_t)c, (c >> 32) != 0 ? ~0u : 0u, k };
}

__device__ __forceinline__ NarrowCoef narrow_coef(int64_t c)
{
    int32_t lo = (int32_t)(uint32_t)(uint64_t)c;
    int32_t hi = (int32_t)((c - (int64_t)lo) >> 32);
    // signs the optimiser could prove are hidden, so that each product stays
    // one signed 32 x 32 -> 64-bit multiply-add
    asm("" : "+v"(lo), "+v"(hi));
    return NarrowCoef{ hi, lo };
}

template <int DIM, int E>
__device__ __forceinline__ BiasedAxis biased_axis(const AxisCoef &c)
{
    return BiasedAxis{ biased_coef<DIM, E>(c.w0), biased_coef<DIM, E>(c.w2), narrow_coef(c.u0),
                       narrow_coef(c.u2) };
}

// HALF: the wavefront holds a weight of exactly one half (only w_0 can be).
template <bool HALF>
__device__ __forceinline__ uint32_t biased_weight_share(uint32_t q, BiasedCoef w)
{
    const uint64_t u = (uint64_t)q * w.c + w.k;
    uint32_t hi = (uint32_t)(u >> 32);
    if constexpr (HALF)
        hi += q & w.half;
    const uint32_t t = (hi & 3u) | (uint32_t)u;
    return (hi - 1u + (t < 1u ? t : 1u)) >> 1;
}

// round-half-even(q c / 2^49) + BOUT for a plain q and a first moment c: with
// u = q lo + 2^48 + 2^49 and V' = q hi + floor(u / 2^32) (two signed
// multiply-adds), q c + 2^48 + 2^49 = 2^32 V' + (u mod 2^32) and V' = V + 2^17
// with V that of q c + 2^48; V' / 2^17 - 1 is the quotient rounded half up,
// and a tie (low word 0, V' = 0 mod 2^18: the rounded-up quotient odd) steps
// down: V' / 2^17 + BOUT - 2 + min(t, 1) with t zero exactly then.
template <uint32_t BOUT>
__device__ __forceinline__ uint32_t biased_moment_share(int32_t q, NarrowCoef c)
{
    // the offset's value is hidden from the optimiser, which would otherwise
    // rewrite the tie test as a separate low-word multiply
    int64_t half = 3ll << 48;
    asm("" : "+s"(half));
    const int64_t u = (int64_t)q * c.lo + half;
    const uint32_t u_lo = (uint32_t)(uint64_t)u;
    const int64_t V = (int64_t)q * c.hi + (u >> 32);
    const uint32_t r = (uint32_t)(uint64_t)(V >> 17);
    const uint32_t t = ((uint32_t)(uint64_t)V & 0x3FFFFu) | u_lo;
    return r + (BOUT - 2u) + (t < 1u ? t : 1u);
}

// The one-axis split of the narrow path: KIND 0 with the weights, KIND 1
// with the first moments; q biased by BIN, its shares by BOUT.
template <int KIND, uint32_t BIN, uint32_t BOUT, bool HALF>
__device__ __forceinline__ void split_biased(uint32_t q, const BiasedAxis &c, uint32_t s[3])
{
    if constexpr (KIND == 0) {
        s[0] = biased_weight_share<HALF>(q, c.w0);
        s[2] = biased_weight_share<false>(q, c.w2);
        s[1] = q - s[0] - s[2];
    } else {
        const int32_t plain = (int32_t)(q - BIN);
        s[0] = biased_moment_share<BOUT>(plain, c.u0);
        s[2] = biased_moment_share<BOUT>(plain, c.u2);
        s[1] = 3u * BOUT - s[0] - s[2];
    }
}

// acc[(a * 3 + b) * 3 + c] (2D: acc[a * 3 + b]) += the biased tensor split
// of the plain q, along x with KX, then y with KY, then z with KZ.
template <int DIM, int KX, int KY, int KZ, bool HALF>
__device__ __forceinline__ void tensor_add_biased(int32_t q, const BiasedAxis (&ax)[DIM],
                                                  uint32_t (&acc)[DIM == 3 ? 27 : 9])
{
    constexpr uint32_t b0 = axis_bias<DIM, 0>(), b1 = axis_bias<DIM, 1>(), b2 = axis_bias<DIM, 2>();
    uint32_t sx[3];
    split_biased<KX, b0, b1, HALF>((uint32_t)q + b0, ax[0], sx);
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        uint32_t sy[3];
        split_biased<KY, b1, b2, HALF>(sx[a], ax[1], sy);
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            if constexpr (DIM == 3) {
                uint32_t sz[3];
                split_biased<KZ, b2, axis_bias<DIM, 3>(), HALF>(sy[b], ax[2], sz);
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    acc[(a * 3 + b) * 3 + c] += sz[c];
            } else {
                acc[a * 3 + b] += sy[b];
            }
        }
    }
}

// Split q along one axis (the wide path): KIND 0 with the weights, KIND 1
// with the first moments; the products formed exactly in 128 bits.
template <int KIND>
__device__ __forceinline__ void split1(int64_t q, const AxisCoef &c, int64_t s[3])
{
    if constexpr (KIND == 0) {
        s[0] = round_shift<33>((__int128)q * c.w0);
        s[2] = round_shift<33>((__int128)q * c.w2);
        s[1] = q - s[0] - s[2];
    } else {
        s[0] = round_shift<49>((__int128)q * c.u0);
        s[2] = round_shift<49>((__int128)q * c.u2);
        s[1] = -s[0] - s[2];
    }
}

// acc[(a * 3 + b) * 3 + c] (2D: acc[a * 3 + b]) += the tensor split of q,
// along x with KX, then y with KY, then z with KZ, with 128-bit products.
template <int DIM, int KX, int KY, int KZ>
__device__ __forceinline__ void tensor_add(int64_t q, const AxisCoef (&ax)[DIM], int64_t (&acc)[DIM == 3 ? 27 : 9])
{
    int64_t sx[3];
    split1<KX>(q, ax[0], sx);
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        int64_t sy[3];
        split1<KY>(sx[a], ax[1], sy);
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            if constexpr (DIM == 3) {
                int64_t sz[3];
                split1<KZ>(sy[b], ax[2], sz);
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    acc[(a * 3 + b) * 3 + c] += sz[c];
            } else {
                acc[a * 3 + b] += sy[b];
            }
        }
    }
}

template <int DIM, class T>
__device__ __forceinline__ void flush(int64_t *g, const T (&acc)[DIM == 3 ? 27 : 9], const int64_t (&base)[DIM],
                                      int64_t n)
{
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int c = 0; c < (DIM == 3 ? 3 : 1); ++c) {
                int64_t node;
                T s;
                if constexpr (DIM == 3) {
                    node = ((base[2] + c) * n + (base[1] + b)) * n + (base[0] + a);
                    s = acc[(a * 3 + b) * 3 + c];
                } else {
                    node = (base[1] + b) * n + (base[0] + a);
                    s = acc[a * 3 + b];
                }
                if (s != 0)
                    atomicAdd(reinterpret_cast<unsigned long long *>(&g[node]), (unsigned long long)(int64_t)s);
            }
}

// Stencil of one particle: base node and split coefficients per axis;
// false when a stencil node leaves [0, n).
template <int DIM>
__device__ __forceinline__ bool stencil(const int32_t *__restrict__ X, int64_t np, int64_t p, int n,
                                        int64_t (&base)[DIM], AxisCoef (&ax)[DIM])
{
    bool inside = true;
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        const int64_t x = X[(int64_t)e * np + p];
        base[e] = (x - 32768) >> 16;                     // floor((x - 2^15) / 2^16)
        inside &= base[e] >= 0 && base[e] <= n - 3;
        ax[e] = axis_coef(x - (base[e] << 16));
    }
    return inside;
}

// Loads m, v, C of particle p; false when one leaves the declared ranges.
template <int DIM>
__device__ __forceinline__ bool load_quantities(const int64_t *__restrict__ m, const int64_t *__restrict__ v,
                                                const int64_t *__restrict__ C, int64_t np, int64_t p,
                                                int64_t max_mass, int64_t max_speed, int64_t max_affine,
                                                int64_t &mp, int64_t (&vp)[DIM], int64_t (&cp)[DIM][DIM])
{
    mp = m[p];
    bool in_range = mp >= -max_mass && mp <= max_mass;
#pragma unroll
    for (int d = 0; d < DIM; ++d) {
        vp[d] = v[(int64_t)d * np + p];
        in_range &= vp[d] >= -max_speed && vp[d] <= max_speed;
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            cp[d][e] = C[(int64_t)(d * DIM + e) * np + p];
            in_range &= cp[d][e] >= -max_affine && cp[d][e] <= max_affine;
        }
    }
    return in_range;
}

// All channels of one particle: sink(channel, acc) receives the 3^dim shares
// of each channel in turn.  NARROW: every quantity m, m v_d, m C_de is below
// 2^28 in magnitude (the declared ranges guarantee it), so every share and
// every node's sum of up to four tensors' shares fits in 32 bits, and the
// biased 32-bit splits apply; otherwise 64-bit shares and 128-bit products.
template <int DIM, bool HALF, class Sink>
__device__ __forceinline__ void particle_shares_narrow(const AxisCoef (&ax)[DIM], int64_t mp,
                                                       const int64_t (&vp)[DIM], const int64_t (&cp)[DIM][DIM],
                                                       Sink &sink)
{
    constexpr int K = DIM == 3 ? 27 : 9;
    BiasedAxis c[DIM];
    c[0] = biased_axis<DIM, 0>(ax[0]);
    c[1] = biased_axis<DIM, 1>(ax[1]);
    if constexpr (DIM == 3)
        c[2] = biased_axis<DIM, 2>(ax[2]);
    uint32_t acc[K];
    int32_t out[K];
#pragma unroll
    for (int i = 0; i < K; ++i)
        acc[i] = 0u - kShareBias;
    tensor_add_biased<DIM, 0, 0, 0, HALF>((int32_t)mp, c, acc);
#pragma unroll
    for (int i = 0; i < K; ++i)
        out[i] = (int32_t)acc[i];
    sink(0, out);
#pragma unroll 1
    for (int d = 0; d < DIM; ++d) {
#pragma unroll
        for (int i = 0; i < K; ++i)
            acc[i] = 0u - (uint32_t)(1 + DIM) * kShareBias;
        // the products are below 2^28, so 32-bit multiplies are exact
        const int32_t m32 = (int32_t)mp;
        tensor_add_biased<DIM, 0, 0, 0, HALF>(m32 * (int32_t)vp[d], c, acc);
        tensor_add_biased<DIM, 1, 0, 0, HALF>(m32 * (int32_t)cp[d][0], c, acc);
        tensor_add_biased<DIM, 0, 1, 0, HALF>(m32 * (int32_t)cp[d][1], c, acc);
        if constexpr (DIM == 3)
            tensor_add_biased<DIM, 0, 0, 1, HALF>(m32 * (int32_t)cp[d][2], c, acc);
#pragma unroll
        for (int i = 0; i < K; ++i)
            out[i] = (int32_t)acc[i];
        sink(1 + d, out);
    }
}

template <int DIM, bool NARROW, class Sink>
__device__ __forceinline__ void particle_shares(const AxisCoef (&ax)[DIM], int64_t mp, const int64_t (&vp)[DIM],
                                                const int64_t (&cp)[DIM][DIM], Sink &&sink)
{
    constexpr int K = DIM == 3 ? 27 : 9;
    if constexpr (NARROW) {
        bool half = false;
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            half |= (ax[e].w0 >> 32) != 0;
        if (__builtin_amdgcn_ballot_w64(half) != 0ull)
            particle_shares_narrow<DIM, true>(ax, mp, vp, cp, sink);
        else
            particle_shares_narrow<DIM, false>(ax, mp, vp, cp, sink);
    } else {
        int64_t acc[K];
#pragma unroll
        for (int i = 0; i < K; ++i)
            acc[i] = 0;
        tensor_add<DIM, 0, 0, 0>(mp, ax, acc);
        sink(0, acc);
#pragma unroll 1
        for (int d = 0; d < DIM; ++d) {
#pragma unroll
            for (int i = 0; i < K; ++i)
                acc[i] = 0;
            tensor_add<DIM, 0, 0, 0>(mp * vp[d], ax, acc);
            tensor_add<DIM, 1, 0, 0>(mp * cp[d][0], ax, acc);
            tensor_add<DIM, 0, 1, 0>(mp * cp[d][1], ax, acc);
            if constexpr (DIM == 3)
                tensor_add<DIM, 0, 0, 1>(mp * cp[d][2], ax, acc);
            sink(1 + d, acc);
        }
    }
}

template <int DIM, bool NARROW>
__global__ void __launch_bounds__(256) isplit_kernel(int64_t np, int n, const int32_t *__restrict__ X,
                                                     const int64_t *__restrict__ m, const int64_t *__restrict__ v,
                                                     const int64_t *__restrict__ C,
                                                     const uint32_t *__restrict__ order, int64_t max_mass,
                                                     int64_t max_speed, int64_t max_affine,
                                                     int64_t *__restrict__ grid, uint32_t *__restrict__ status)
{
    const int64_t nodes = DIM == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < np; k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = order ? (int64_t)order[k] : k;
        if (p >= np) {                   // an order entry that names no particle
            atomicAdd(&status[3], 1u);
            continue;
        }
        int64_t base[DIM];
        AxisCoef ax[DIM];
        const bool inside = stencil<DIM>(X, np, p, n, base, ax);
        int64_t mp, vp[DIM], cp[DIM][DIM];
        const bool in_range = load_quantities<DIM>(m, v, C, np, p, max_mass, max_speed, max_affine, mp, vp, cp);
        wave_count(!inside, &status[0]);
        wave_count(inside && !in_range, &status[1]);
        if (!inside || !in_range)
            continue;
        particle_shares<DIM, NARROW>(ax, mp, vp, cp, [&](int ch, const auto &acc) {
            flush<DIM>(grid + ch * nodes, acc, base, n);
        });
    }
}

// ---------------------------------------------------------------------------
// Tiled path.
// ---------------------------------------------------------------------------
// A particle's tile-ordered copy: position and quantities in one record,
// written by the scatter in tile order so that the accumulating kernel
// streams whole lines instead of gathering 4 to 8 bytes from each of the
// caller's 16 arrays per particle.  The wide path keeps 64-bit quantities in
// 128 bytes (one cache line); the narrow path, whose quantities the scatter
// has range-checked (so they fit in 32 bits), 32-bit ones in 64 bytes.
struct __align__(16) IsRecord {
    int32_t X[4];          // X[DIM..3] unused
    int64_t m;
    int64_t v[3];          // v[DIM..2] unused
    int64_t C[9];          // (d, e) at d * DIM + e
    int64_t pad;
};
static_assert(sizeof(IsRecord) == 128, "one record per 128-byte line");

struct __align__(16) IsRecord32 {
    int32_t X[3];          // X[DIM..2] unused
    int32_t m;
    int32_t v[3];          // v[DIM..2] unused
    int32_t C[9];          // (d, e) at d * DIM + e
};
static_assert(sizeof(IsRecord32) == 64, "two records per 128-byte line");

template <bool NARROW>
using IsRec = typename std::conditional<NARROW, IsRecord32, IsRecord>::type;

constexpr int kIsTile = 8;                 // cells per tile edge
constexpr int kIsBlock = kIsTile + 2;      // nodes per block edge: bases t0..t0+7 reach t0..t0+9
constexpr int kIsChunk = 2048;             // particles per work item
constexpr int kIsThreads = 256;
constexpr int kScanPer = 4;                // scan entries per thread
constexpr int kScanBlock = kIsThreads * kScanPer;

template <int DIM>
__device__ __forceinline__ int64_t tile_of(const int64_t (&base)[DIM], int64_t tx)
{
    int64_t t = 0;
#pragma unroll
    for (int e = DIM - 1; e >= 0; --e)
        t = t * tx + base[e] / kIsTile;
    return t;
}

__global__ void __launch_bounds__(256) is_zero_kernel(uint32_t *__restrict__ a, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
        a[i] = 0u;
}

// Tile of every visited particle; its rank among the particles of its
// counter comes from the returning atomic on that counter.  Each tile has
// 2^sshift counters (slots), laid out tile-major; visit k uses slot
// (k / 256) mod 2^sshift, which spreads the atomics on one tile over several
// addresses.  Particles whose stencil leaves the grid get rank ~0 and are
// counted; the range check is the accumulating kernel's.
template <int DIM>
__global__ void __launch_bounds__(256) is_count_kernel(int64_t np, int n, int64_t tx, int sshift,
                                                       const int32_t *__restrict__ X,
                                                       const uint32_t *__restrict__ order,
                                                       uint32_t *__restrict__ count, uint32_t *__restrict__ rank,
                                                       uint32_t *__restrict__ status)
{
    const int64_t smask = (1ll << sshift) - 1;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < np; k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = order ? (int64_t)order[k] : k;
        uint32_t r = ~0u;
        bool inside = false;
        if (p >= np) {
            atomicAdd(&status[3], 1u);
            inside = true;               // not a stencil fault
        } else {
            int64_t base[DIM];
            AxisCoef ax[DIM];
            inside = stencil<DIM>(X, np, p, n, base, ax);
            if (inside)
                r = atomicAdd(&count[(tile_of<DIM>(base, tx) << sshift) | ((k >> 8) & smask)], 1u);
        }
        wave_count(!inside, &status[0]);
        rank[k] = r;
    }
}

// Particles of tile t: the sum of its slot counters.
__device__ __forceinline__ uint64_t tile_total(const uint32_t *__restrict__ count, int64_t t, int sshift)
{
    uint64_t c = 0;
    for (int q = 0; q < (1 << sshift); ++q)
        c += count[(t << sshift) + q];
    return c;
}

// Packed scan entry e (tile e >> sshift, slot e mod 2^sshift): particles of
// the slot in the low word; on the tile's last slot, the tile's work items in
// the high word.  Totals stay below 2^32, so neither half carries into the
// other; the exclusive scan at a tile's first slot holds the items and
// particles of all tiles before it.
__device__ __forceinline__ uint64_t packed_entry(const uint32_t *__restrict__ count, int64_t e, int64_t entries,
                                                 int sshift)
{
    if (e >= entries)
        return 0ull;
    const uint64_t c = count[e];
    const int64_t smask = (1ll << sshift) - 1;
    if ((e & smask) != smask)
        return c;
    const uint64_t total = tile_total(count, e >> sshift, sshift);
    return (((total + kIsChunk - 1) / kIsChunk) << 32) | c;
}

// Exclusive scan of 256 threads' values; returns the block total in *total.
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t x, uint64_t *lds_waves, uint64_t *total)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    uint64_t inc = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t o = __shfl_up(inc, d, kWave);
        if (lane >= d)
            inc += o;
    }
    if (lane == kWave - 1)
        lds_waves[wave] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kIsThreads / kWave; ++w) {
        const uint64_t s = lds_waves[w];
        before += w < wave ? s : 0ull;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

__global__ void __launch_bounds__(kIsThreads) is_scan_partial_kernel(const uint32_t *__restrict__ count,
                                                                     int64_t entries, int sshift,
                                                                     uint64_t *__restrict__ partial)
{
    __shared__ uint64_t lw[kIsThreads / kWave];
    const int64_t t0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPer;
    uint64_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i)
        s += packed_entry(count, t0 + i, entries, sshift);
    uint64_t total;
    block_exclusive_scan(s, lw, &total);
    if (threadIdx.x == 0)
        partial[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the block totals in place; meta[0] = the
// grand total (items << 32 | particles).
__global__ void __launch_bounds__(kIsThreads) is_scan_top_kernel(uint64_t *__restrict__ partial, int64_t blocks,
                                                                 uint64_t *__restrict__ meta)
{
    __shared__ uint64_t lw[kIsThreads / kWave];
    uint64_t carry = 0;
    for (int64_t b0 = 0; b0 < blocks; b0 += kIsThreads) {
        const int64_t b = b0 + threadIdx.x;
        const uint64_t x = b < blocks ? partial[b] : 0ull;
        uint64_t total;
        const uint64_t ex = block_exclusive_scan(x, lw, &total);
        if (b < blocks)
            partial[b] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0)
        meta[0] = carry;
}

__global__ void __launch_bounds__(kIsThreads) is_scan_final_kernel(const uint32_t *__restrict__ count,
                                                                   int64_t entries, int sshift,
                                                                   const uint64_t *__restrict__ partial,
                                                                   uint64_t *__restrict__ start)
{
    __shared__ uint64_t lw[kIsThreads / kWave];
    const int64_t t0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPer;
    uint64_t e[kScanPer], s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        e[i] = packed_entry(count, t0 + i, entries, sshift);
        s += e[i];
    }
    uint64_t total;
    uint64_t run = partial[blockIdx.x] + block_exclusive_scan(s, lw, &total);
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        if (t0 + i < entries)
            start[t0 + i] = run;
        run += e[i];
    }
}

// Each visited particle's record goes to its tile's range at its rank.
// NARROW: the declared ranges are checked here (a particle outside them is
// counted in status[1] and its record carries zero mass, velocity and affine
// matrix, so it adds nothing), and the quantities are stored in 32 bits.
template <int DIM, bool NARROW>
__global__ void __launch_bounds__(256) is_scatter_kernel(int64_t np, int n, int64_t tx, int sshift,
                                                         const int32_t *__restrict__ X,
                                                         const int64_t *__restrict__ m,
                                                         const int64_t *__restrict__ v,
                                                         const int64_t *__restrict__ C,
                                                         const uint32_t *__restrict__ order,
                                                         const uint32_t *__restrict__ rank,
                                                         const uint64_t *__restrict__ start, int64_t max_mass,
                                                         int64_t max_speed, int64_t max_affine,
                                                         IsRec<NARROW> *__restrict__ rec,
                                                         uint32_t *__restrict__ status)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < np; k += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t r = rank[k];
        const bool visit = r != ~0u;
        const int64_t p = order ? (int64_t)order[k] : k;
        int64_t base[DIM];
        AxisCoef ax[DIM];
        if (visit)
            stencil<DIM>(X, np, p, n, base, ax);
        IsRec<NARROW> q;
        if (visit) {
#pragma unroll
            for (int d = 0; d < (NARROW ? 3 : 4); ++d)
                q.X[d] = d < DIM ? X[(int64_t)d * np + p] : 0;
        }
        if constexpr (NARROW) {
            int64_t mp = 0, vp[DIM], cp[DIM][DIM];
            bool in_range = true;
            if (visit)
                in_range = load_quantities<DIM>(m, v, C, np, p, max_mass, max_speed, max_affine, mp, vp, cp);
            wave_count(visit && !in_range, &status[1]);
            if (!visit)
                continue;
            q.m = in_range ? (int32_t)mp : 0;
#pragma unroll
            for (int d = 0; d < 3; ++d)
                q.v[d] = d < DIM && in_range ? (int32_t)vp[d < DIM ? d : 0] : 0;
#pragma unroll
            for (int i = 0; i < 9; ++i)
                q.C[i] = i < DIM * DIM && in_range ? (int32_t)cp[(i < DIM * DIM ? i : 0) / DIM][(i < DIM * DIM ? i : 0) % DIM]
                                                   : 0;
        } else {
            if (!visit)
                continue;
            q.m = m[p];
#pragma unroll
            for (int d = 0; d < 3; ++d)
                q.v[d] = d < DIM ? v[(int64_t)d * np + p] : 0;
#pragma unroll
            for (int i = 0; i < 9; ++i)
                q.C[i] = i < DIM * DIM ? C[(int64_t)i * np + p] : 0;
            q.pad = 0;
        }
        const int64_t e = (tile_of<DIM>(base, tx) << sshift) | ((k >> 8) & ((1ll << sshift) - 1));
        constexpr int W = (int)(sizeof(IsRec<NARROW>) / 16);
        const uint4 *src = reinterpret_cast<const uint4 *>(&q);
        uint4 *dst = reinterpret_cast<uint4 *>(rec + (int64_t)(start[e] & 0xFFFFFFFFull) + r);
#pragma unroll
        for (int w = 0; w < W; ++w)
            dst[w] = src[w];
    }
}

// Work item i -> the tile whose items contain it: the last tile whose first
// item is <= i (an empty tile shares its first item with the next tile, so
// the last such tile is never empty).
__device__ __forceinline__ int64_t item_tile(const uint64_t *__restrict__ start, int64_t tiles, int sshift,
                                             uint64_t i)
{
    int64_t lo = 0, hi = tiles;          // first tile with first item > i lies in (lo, hi]
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if ((start[mid << sshift] >> 32) <= i)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

typedef __attribute__((address_space(3))) unsigned long long lds_u64;

template <int DIM, bool NARROW>
__global__ void __launch_bounds__(kIsThreads) is_tiled_kernel(int64_t np, int n, int64_t tx, int64_t tiles, int sshift,
                                                              const IsRec<NARROW> *__restrict__ rec,
                                                              const uint32_t *__restrict__ count,
                                                              const uint64_t *__restrict__ start,
                                                              const uint64_t *__restrict__ meta, int64_t max_mass,
                                                              int64_t max_speed, int64_t max_affine,
                                                              int64_t *__restrict__ grid,
                                                              uint32_t *__restrict__ status)
{
    constexpr int B = kIsBlock;
    constexpr int plane = DIM == 3 ? B * B * B : B * B;
    constexpr int entries = (1 + DIM) * plane;
    __shared__ unsigned long long block[entries];
    const int64_t nodes = DIM == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const uint64_t items = meta[0] >> 32;
    for (uint64_t i = blockIdx.x; i < items; i += gridDim.x) {
        const int64_t t = item_tile(start, tiles, sshift, i);
        const uint64_t s = start[t << sshift];
        const int64_t lo = (int64_t)(s & 0xFFFFFFFFull) + (int64_t)(i - (s >> 32)) * kIsChunk;
        const int64_t end_t = (int64_t)(s & 0xFFFFFFFFull) + (int64_t)tile_total(count, t, sshift);
        const int64_t hi = lo + kIsChunk < end_t ? lo + kIsChunk : end_t;
        int64_t origin[DIM];
        {
            int64_t r = t;
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                origin[e] = (r % tx) * kIsTile;
                r /= tx;
            }
        }
        for (int e = threadIdx.x; e < entries; e += kIsThreads)
            block[e] = 0ull;
        __syncthreads();
        for (int64_t j = lo + threadIdx.x; j < hi; j += kIsThreads) {
            IsRec<NARROW> q;
            {
                constexpr int W = (int)(sizeof(IsRec<NARROW>) / 16);
                const uint4 *src = reinterpret_cast<const uint4 *>(rec + j);
                uint4 *dst = reinterpret_cast<uint4 *>(&q);
#pragma unroll
                for (int w = 0; w < W; ++w)
                    dst[w] = src[w];
            }
            int64_t base[DIM];
            AxisCoef ax[DIM];
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                const int64_t x = q.X[e];
                base[e] = (x - 32768) >> 16;
                ax[e] = axis_coef(x - (base[e] << 16));
            }
            const int64_t mp = q.m;
            int64_t vp[DIM], cp[DIM][DIM];
            bool in_range = mp >= -max_mass && mp <= max_mass;
#pragma unroll
            for (int d = 0; d < DIM; ++d) {
                vp[d] = q.v[d];
                in_range &= vp[d] >= -max_speed && vp[d] <= max_speed;
#pragma unroll
                for (int e = 0; e < DIM; ++e) {
                    cp[d][e] = q.C[d * DIM + e];
                    in_range &= cp[d][e] >= -max_affine && cp[d][e] <= max_affine;
                }
            }
            if constexpr (!NARROW) {         // (narrow: checked by the scatter)
                wave_count(!in_range, &status[1]);
                if (!in_range)
                    continue;
            }
            int lb[DIM];
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                lb[e] = (int)(base[e] - origin[e]);
            particle_shares<DIM, NARROW>(ax, mp, vp, cp, [&](int ch, const auto &acc) {
                // the stencil's first node in the block, formed once: its 27
                // (9) nodes are fixed offsets from it, which the LDS atomics
                // carry as immediates (left to itself the compiler rebuilds
                // the address inside every conditional add)
                lds_u64 *nb = (lds_u64 *)&block[DIM == 3 ? ((ch * B + lb[DIM - 1]) * B + lb[1]) * B + lb[0]
                                                         : (ch * B + lb[1]) * B + lb[0]];
                asm volatile("" : "+v"(nb));
#pragma unroll
                for (int a = 0; a < 3; ++a)
#pragma unroll
                    for (int b = 0; b < 3; ++b)
#pragma unroll
                        for (int c = 0; c < (DIM == 3 ? 3 : 1); ++c) {
                            int off;
                            int64_t sh;      // a 32-bit share widened with its sign
                            if constexpr (DIM == 3) {
                                off = (c * B + b) * B + a;
                                sh = acc[(a * 3 + b) * 3 + c];
                            } else {
                                off = b * B + a;
                                sh = acc[a * 3 + b];
                            }
                            if (sh != 0)
                                __hip_atomic_fetch_add(nb + off, (unsigned long long)sh, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
            });
        }
        __syncthreads();
        for (int e = threadIdx.x; e < entries; e += kIsThreads) {
            const unsigned long long val = block[e];
            if (val == 0ull)
                continue;
            const int ch = e / plane;
            int r = e - ch * plane;
            const int lx = r % B;
            r /= B;
            int64_t node;
            bool ok;
            if constexpr (DIM == 3) {
                const int ly = r % B, lz = r / B;
                const int64_t x = origin[0] + lx, y = origin[1] + ly, z = origin[2] + lz;
                ok = x < n && y < n && z < n;
                node = (z * n + y) * n + x;
            } else {
                const int64_t x = origin[0] + lx, y = origin[1] + r;
                ok = x < n && y < n;
                node = y * n + x;
            }
            if (ok)
                atomicAdd(reinterpret_cast<unsigned long long *>(&grid[ch * nodes + node]), val);
        }
        __syncthreads();
    }
}

// The narrow path needs every split quantity m, m v_d, m C_de below 2^28 in
// magnitude: max_mass * max(1, max_speed, max_affine) < 2^28 (particles
// beyond the declared ranges are skipped).  A share of q is then at most
// 3/4 |q| + 1 in magnitude (the weights are at most 3/4, the first moments
// at most 1/4 in magnitude, and a near share adds the two roundings of the
// outer ones), so the values entering each axis' splits stay below 2^28 + 2
// and a node's sum over the four tensors of a momentum channel below
// 4 (2^28 + 3) < 2^31: 32-bit values and sums throughout, and products of
// 29 by 49 bits in two 32 x 32 -> 64-bit multiply-adds.
bool narrow_ranges(int64_t max_mass, int64_t max_speed, int64_t max_affine)
{
    int64_t f = max_speed > max_affine ? max_speed : max_affine;
    f = f > 1 ? f : 1;
    return (__int128)max_mass * f < ((__int128)1 << 28);
}

int64_t is_blocks(int64_t work, int64_t cap_per_cu)
{
    const int64_t want = (work + 255) / 256, cap = (int64_t)device_cu_count() * cap_per_cu;
    return want < 1 ? 1 : (want > cap ? cap : want);
}

// The tiled path's workspace for callers that cannot allocate
// (mpm_p2g_isplit_noalloc): a file-scope device array, one per GPU, held
// until the process ends.  In host code `scratch` only names the symbol;
// its device address comes from hipGetSymbolAddress (isplit_scratch below).
__device__ __align__(256) uint8_t scratch[MPM_ISPLIT_SCRATCH_BYTES];

}  // namespace

IsplitLayout isplit_layout(int dim, int n, int64_t np)
{
    IsplitLayout l{};
    l.tiles_x = (n - 2 + kIsTile - 1) / kIsTile;           // bases 0..n-3
    l.tiles = dim == 3 ? l.tiles_x * l.tiles_x * l.tiles_x : l.tiles_x * l.tiles_x;
    l.slot_shift = 3;                                      // up to 8 counters per tile, at most 2^22 in all
    while (l.slot_shift > 0 && (l.tiles << l.slot_shift) > (1ll << 22))
        --l.slot_shift;
    l.entries = l.tiles << l.slot_shift;
    l.scan_blocks = (l.entries + kScanBlock - 1) / kScanBlock;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    l.count = take(sizeof(uint32_t) * (size_t)l.entries);
    l.start = take(sizeof(uint64_t) * (size_t)l.entries);
    l.partial = take(sizeof(uint64_t) * (size_t)l.scan_blocks);
    l.meta = take(sizeof(uint64_t) * 2);
    l.rank = take(sizeof(uint32_t) * (size_t)(np > 0 ? np : 1));
    l.rec = take(sizeof(IsRecord) * (size_t)(np > 0 ? np : 1));
    l.total = off;
    return l;
}

hipError_t launch_p2g_isplit_tiled(int dim, int n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                                   const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                                   int64_t max_affine, void *ws, int64_t *grid, uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const IsplitLayout l = isplit_layout(dim, n, np);
    char *w = static_cast<char *>(ws);
    uint32_t *count = reinterpret_cast<uint32_t *>(w + l.count);
    uint64_t *start = reinterpret_cast<uint64_t *>(w + l.start);
    uint64_t *partial = reinterpret_cast<uint64_t *>(w + l.partial);
    uint64_t *meta = reinterpret_cast<uint64_t *>(w + l.meta);
    uint32_t *rank = reinterpret_cast<uint32_t *>(w + l.rank);
    const dim3 blk(kIsThreads);
    const int sh = l.slot_shift;
    hipLaunchKernelGGL(is_zero_kernel, dim3((unsigned)is_blocks(l.entries, 16)), blk, 0, s, count, l.entries);
    const unsigned pb = (unsigned)is_blocks(np, 32);
    if (dim == 3)
        hipLaunchKernelGGL(is_count_kernel<3>, dim3(pb), blk, 0, s, np, n, l.tiles_x, sh, X, order, count, rank,
                           status);
    else
        hipLaunchKernelGGL(is_count_kernel<2>, dim3(pb), blk, 0, s, np, n, l.tiles_x, sh, X, order, count, rank,
                           status);
    hipLaunchKernelGGL(is_scan_partial_kernel, dim3((unsigned)l.scan_blocks), blk, 0, s, count, l.entries, sh,
                       partial);
    hipLaunchKernelGGL(is_scan_top_kernel, dim3(1), blk, 0, s, partial, l.scan_blocks, meta);
    hipLaunchKernelGGL(is_scan_final_kernel, dim3((unsigned)l.scan_blocks), blk, 0, s, count, l.entries, sh, partial,
                       start);
    const bool narrow = narrow_ranges(max_mass, max_speed, max_affine);
    auto scatter = [&](auto kern, auto *records) {
        hipLaunchKernelGGL(kern, dim3(pb), blk, 0, s, np, n, l.tiles_x, sh, X, m, v, C, order, rank, start, max_mass,
                           max_speed, max_affine, records, status);
    };
    IsRecord *rec = reinterpret_cast<IsRecord *>(w + l.rec);
    IsRecord32 *rec32 = reinterpret_cast<IsRecord32 *>(w + l.rec);
    if (dim == 3)
        narrow ? scatter(is_scatter_kernel<3, true>, rec32) : scatter(is_scatter_kernel<3, false>, rec);
    else
        narrow ? scatter(is_scatter_kernel<2, true>, rec32) : scatter(is_scatter_kernel<2, false>, rec);
    // items <= tiles + np / kIsChunk; persistent workgroups stride over them
    const int64_t max_items = l.tiles + np / kIsChunk + 1;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    const unsigned tb = (unsigned)(max_items < cap ? max_items : cap);
auto tiled = [&](auto kern, auto *records) {
        hipLaunchKernelGGL(kern, dim3(tb), blk, 0, s, np, n, l.tiles_x, l.tiles, sh, records, count, start, meta,
                           max_mass, max_speed, max_affine, grid, status);
    };
    if (dim == 3)
        narrow ? tiled(is_tiled_kernel<3, true>, rec32) : tiled(is_tiled_kernel<3, false>, rec);
    else
        narrow ? tiled(is_tiled_kernel<2, true>, rec32) : tiled(is_tiled_kernel<2, false>, rec);
    return hipGetLastError();
}

hipError_t launch_p2g_isplit(int dim, int n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                             const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                             int64_t max_affine, int64_t *grid, uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const int64_t want = (np + 255) / 256, cap = (int64_t)device_cu_count() * 32;
    const int blocks = (int)(want > cap ? cap : want);
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, np, n, X, m, v, C, order, max_mass, max_speed,
                           max_affine, grid, status);
    };
    const bool narrow = narrow_ranges(max_mass, max_speed, max_affine);
    if (dim == 3)
        narrow ? launch(isplit_kernel<3, true>) : launch(isplit_kernel<3, false>);
    else
        narrow ? launch(isplit_kernel<2, true>) : launch(isplit_kernel<2, false>);
    return hipGetLastError();
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current and kept; every later call on the device reuses
// it.  Returns the lookup's error (and leaves *ptr NULL) on failure.
hipError_t isplit_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace mpmk
