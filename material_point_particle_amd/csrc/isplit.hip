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
// One thread per particle; its 3^dim shares of one channel are formed in
// registers and added with one 64-bit global atomic each.  Integer atomics
// commute, so the grid is bit-identical in every order and every launch.
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

// Split q along one axis: KIND 0 with the weights, KIND 1 with the first moments.
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
// along x with KX, then y with KY, then z with KZ.
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

template <int DIM>
__device__ __forceinline__ void flush(int64_t *g, const int64_t (&acc)[DIM == 3 ? 27 : 9], const int64_t (&base)[DIM],
                                      int64_t n)
{
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int c = 0; c < (DIM == 3 ? 3 : 1); ++c) {
                int64_t node, s;
                if constexpr (DIM == 3) {
                    node = ((base[2] + c) * n + (base[1] + b)) * n + (base[0] + a);
                    s = acc[(a * 3 + b) * 3 + c];
                } else {
                    node = (base[1] + b) * n + (base[0] + a);
                    s = acc[a * 3 + b];
                }
                if (s != 0)
                    atomicAdd(reinterpret_cast<unsigned long long *>(&g[node]), (unsigned long long)s);
            }
}

template <int DIM>
__global__ void __launch_bounds__(256) isplit_kernel(int64_t np, int n, const int32_t *__restrict__ X,
                                                     const int64_t *__restrict__ m, const int64_t *__restrict__ v,
                                                     const int64_t *__restrict__ C,
                                                     const uint32_t *__restrict__ order, int64_t max_mass,
                                                     int64_t max_speed, int64_t max_affine,
                                                     int64_t *__restrict__ grid, uint32_t *__restrict__ status)
{
    constexpr int K = DIM == 3 ? 27 : 9;
    const int64_t nodes = DIM == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < np; k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = order ? (int64_t)order[k] : k;
        if (p >= np) {                   // an order entry that names no particle
            atomicAdd(&status[3], 1u);
            continue;
        }
        int64_t base[DIM];
        AxisCoef ax[DIM];
        bool inside = true;
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            const int64_t x = X[(int64_t)e * np + p];
            base[e] = (x - 32768) >> 16;                 // floor((x - 2^15) / 2^16)
            inside &= base[e] >= 0 && base[e] <= n - 3;
            ax[e] = axis_coef(x - (base[e] << 16));
        }
        const int64_t mp = m[p];
        bool in_range = mp >= -max_mass && mp <= max_mass;
        int64_t vp[DIM], cp[DIM][DIM];
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
        wave_count(!inside, &status[0]);
        wave_count(inside && !in_range, &status[1]);
        if (!inside || !in_range)
            continue;

        int64_t acc[K];
#pragma unroll
        for (int i = 0; i < K; ++i)
            acc[i] = 0;
        tensor_add<DIM, 0, 0, 0>(mp, ax, acc);
        flush<DIM>(grid, acc, base, n);
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
            flush<DIM>(grid + (1 + d) * nodes, acc, base, n);
        }
    }
}

}  // namespace

hipError_t launch_p2g_isplit(int dim, int n, int64_t np, const int32_t *X, const int64_t *m, const int64_t *v,
                             const int64_t *C, const uint32_t *order, int64_t max_mass, int64_t max_speed,
                             int64_t max_affine, int64_t *grid, uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const int64_t want = (np + 255) / 256, cap = (int64_t)device_cu_count() * 32;
    const int blocks = (int)(want > cap ? cap : want);
    if (dim == 3)
        hipLaunchKernelGGL(isplit_kernel<3>, dim3(blocks), dim3(256), 0, s, np, n, X, m, v, C, order, max_mass,
                           max_speed, max_affine, grid, status);
    else
        hipLaunchKernelGGL(isplit_kernel<2>, dim3(blocks), dim3(256), 0, s, np, n, X, m, v, C, order, max_mass,
                           max_speed, max_affine, grid, status);
    return hipGetLastError();
}

}  // namespace mpmk
