// stress.hip -- MLS-MPM stress term of a Neo-Hookean solid, and the
// deformation-gradient update.
//
// "Implementation -- GPU Optimization & Reference Codebases", section 3.1,
// part 2 of the guide described there: with J = det F and F^-T = (F^T)^-1,
// P = mu (F - F^-T) + lambda log(J) F^-T and sigma = (1/J) P F^T.  The stress
// enters the MLS-MPM transfer through the affine term: a particle adds
// w_i (m v + Q (x_i - x_p)) to node i with Q = m C - dt vol sigma D^-1,
// D^-1 = 4 n^2 for the quadratic B-spline and vol sigma = vol0 P F^T.  Divided
// by m, P2G's arithmetic is unchanged when its affine matrix is
//   C' = C - k (P F^T),   k = dt vol0 4 n^2 / m,
// so this is one elementwise pass before binning and P2G, and the P2G kernels
// stay as they are.  After G2P, F <- (I + dt C) F.
//
// Both passes are one thread per particle over component-major arrays
// (coalesced); they are HBM-bound.  The stress is formed in float64 in a fixed
// order and each C' entry is rounded to float32 once.
#include "common.hpp"

namespace mpmk {
namespace {

template <int DIM>
__global__ void __launch_bounds__(256) neohookean_affine_kernel(int64_t np, double scale, const float *__restrict__ F,
                                                                const float *__restrict__ C,
                                                                const float *__restrict__ m,
                                                                const float *__restrict__ vol0, float dt, float mu,
                                                                float lambda, float *__restrict__ Cout,
                                                                uint32_t *__restrict__ status)
{
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        double f[DIM][DIM], cof[DIM][DIM];
        float c[DIM][DIM];
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                f[d][e] = (double)F[(int64_t)(d * DIM + e) * np + p];
                c[d][e] = C[(int64_t)(d * DIM + e) * np + p];
            }
        double J;
        if constexpr (DIM == 3) {
            cof[0][0] = f[1][1] * f[2][2] - f[1][2] * f[2][1];
            cof[0][1] = f[1][2] * f[2][0] - f[1][0] * f[2][2];
            cof[0][2] = f[1][0] * f[2][1] - f[1][1] * f[2][0];
            cof[1][0] = f[0][2] * f[2][1] - f[0][1] * f[2][2];
            cof[1][1] = f[0][0] * f[2][2] - f[0][2] * f[2][0];
            cof[1][2] = f[0][1] * f[2][0] - f[0][0] * f[2][1];
            cof[2][0] = f[0][1] * f[1][2] - f[0][2] * f[1][1];
            cof[2][1] = f[0][2] * f[1][0] - f[0][0] * f[1][2];
            cof[2][2] = f[0][0] * f[1][1] - f[0][1] * f[1][0];
            J = (f[0][0] * cof[0][0] + f[0][1] * cof[0][1]) + f[0][2] * cof[0][2];
        } else {
            cof[0][0] = f[1][1];
            cof[0][1] = -f[1][0];
            cof[1][0] = -f[0][1];
            cof[1][1] = f[0][0];
            J = f[0][0] * f[1][1] - f[0][1] * f[1][0];
        }
        const bool inverted = !(J > 0.0);
        wave_count(inverted, &status[0]);
        float out[DIM][DIM];
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                out[d][e] = c[d][e];
        const float mp = m[p];
        if (!inverted && mp != 0.0f) {
            const double llj = (double)lambda * log(J);
            double P[DIM][DIM];
#pragma unroll
            for (int d = 0; d < DIM; ++d)
#pragma unroll
                for (int e = 0; e < DIM; ++e) {
                    const double fit = cof[d][e] / J;                   // (F^-T)_de
                    P[d][e] = (double)mu * (f[d][e] - fit) + llj * fit;
                }
            const double k = (((double)dt * (double)vol0[p]) * scale) / (double)mp;
#pragma unroll
            for (int d = 0; d < DIM; ++d)
#pragma unroll
                for (int e = 0; e < DIM; ++e) {
                    double tau = 0.0;                                   // (P F^T)_de
#pragma unroll
                    for (int q = 0; q < DIM; ++q)
                        tau = tau + P[d][q] * f[e][q];
                    out[d][e] = (float)((double)c[d][e] - k * tau);
                }
        }
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                Cout[(int64_t)(d * DIM + e) * np + p] = out[d][e];
    }
}

// F <- (I + dt C) F: G_dq = [d == q] + dt C_dq, F'_de = sum_q G_dq F_qe in
// order q = 0, 1, 2, all float32.
template <int DIM>
__global__ void __launch_bounds__(256) update_F_kernel(int64_t np, const float *__restrict__ C, float *__restrict__ F,
                                                       float dt)
{
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        float G[DIM][DIM], f[DIM][DIM];
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int q = 0; q < DIM; ++q) {
                G[d][q] = (d == q ? 1.0f : 0.0f) + dt * C[(int64_t)(d * DIM + q) * np + p];
                f[d][q] = F[(int64_t)(d * DIM + q) * np + p];
            }
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int e = 0; e < DIM; ++e) {
                float t = G[d][0] * f[0][e];
#pragma unroll
                for (int q = 1; q < DIM; ++q)
                    t = t + G[d][q] * f[q][e];
                F[(int64_t)(d * DIM + e) * np + p] = t;
            }
    }
}

int stress_blocks(int64_t np)
{
    const int64_t want = (np + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

hipError_t launch_neohookean_affine(int dim, int n, int64_t np, const float *F, const float *C, const float *m,
                                    const float *vol0, float dt, float mu, float lambda, float *Cout,
                                    uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const double scale = 4.0 * (double)n * (double)n;
    if (dim == 3)
        hipLaunchKernelGGL(neohookean_affine_kernel<3>, dim3(stress_blocks(np)), dim3(256), 0, s, np, scale, F, C, m,
                           vol0, dt, mu, lambda, Cout, status);
    else
        hipLaunchKernelGGL(neohookean_affine_kernel<2>, dim3(stress_blocks(np)), dim3(256), 0, s, np, scale, F, C, m,
                           vol0, dt, mu, lambda, Cout, status);
    return hipGetLastError();
}

hipError_t launch_update_F(int dim, int64_t np, const float *C, float *F, float dt, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    if (dim == 3)
        hipLaunchKernelGGL(update_F_kernel<3>, dim3(stress_blocks(np)), dim3(256), 0, s, np, C, F, dt);
    else
        hipLaunchKernelGGL(update_F_kernel<2>, dim3(stress_blocks(np)), dim3(256), 0, s, np, C, F, dt);
    return hipGetLastError();
}

}  // namespace mpmk
