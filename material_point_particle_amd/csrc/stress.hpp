// stress.hpp -- the per-particle Neo-Hookean stress term and F update
// (used by stress.hip's passes and by the G2P pass that runs them after the
// gather, grid.hip), and the launcher of the one-pass F update with the next
// substep's stressed affine matrix.
#pragma once
#include "common.hpp"

namespace mpmk {

// C' of one particle from its F (float32, as stored) and C: the Neo-Hookean
// stress formed in float64 in a fixed order, each entry rounded to float32
// once.  Returns true when det F <= 0 (C' = C, counted by the caller).
template <int DIM>
__device__ __forceinline__ bool stressed_affine(const float (&fs)[DIM][DIM], const float (&c)[DIM][DIM], float mp,
                                                float vol, double scale, float dt, float mu, float lambda,
                                                float (&out)[DIM][DIM])
{
    double f[DIM][DIM], cof[DIM][DIM];
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            f[d][e] = (double)fs[d][e];
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
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            out[d][e] = c[d][e];
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
        const double k = (((double)dt * (double)vol) * scale) / (double)mp;
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
    return inverted;
}

// F <- (I + dt C) F of one particle: G_dq = [d == q] + dt C_dq,
// F'_de = sum_q G_dq F_qe in order q = 0, 1, 2, all float32.
template <int DIM>
__device__ __forceinline__ void updated_F(const float (&c)[DIM][DIM], float dt, float (&f)[DIM][DIM])
{
    float G[DIM][DIM], g[DIM][DIM];
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int q = 0; q < DIM; ++q) {
            G[d][q] = (d == q ? 1.0f : 0.0f) + dt * c[d][q];
            g[d][q] = f[d][q];
        }
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            float t = G[d][0] * g[0][e];
#pragma unroll
            for (int q = 1; q < DIM; ++q)
                t = t + G[d][q] * g[q][e];
            f[d][e] = t;
        }
}

template <int DIM>
__device__ __forceinline__ void load_mat(const float *__restrict__ a, int64_t np, int64_t p, float (&m)[DIM][DIM])
{
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            m[d][e] = a[(int64_t)(d * DIM + e) * np + p];
}

template <int DIM>
__device__ __forceinline__ void store_mat(float *__restrict__ a, int64_t np, int64_t p, const float (&m)[DIM][DIM])
{
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            a[(int64_t)(d * DIM + e) * np + p] = m[d][e];
}

hipError_t launch_update_F_stress(int dim, int n, int64_t np, const float *C, float *F, const float *m,
                                  const float *vol0, float dt, float mu, float lambda, float *Cout, uint32_t *status,
                                  hipStream_t s);

// G2P of the particles from vg and then launch_update_F_stress's pass, one
// launch (grid.hip).
hipError_t launch_g2p_stress(int dim, int n, const float *vg, float *x, float *v, float *C, int64_t np, float dt,
                             float *F, const float *m, const float *vol0, float mu, float lambda, float *Cout,
                             uint32_t *status, hipStream_t s);

}  // namespace mpmk
