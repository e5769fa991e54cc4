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
// order and each C' entry is rounded to float32 once.  In a substep loop the
// F update and the next substep's C' can run as one pass (the same
// arithmetic, C and F read once).
#include "stress.hpp"

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
        float f[DIM][DIM], c[DIM][DIM], out[DIM][DIM];
        load_mat<DIM>(F, np, p, f);
        load_mat<DIM>(C, np, p, c);
        const bool inverted = stressed_affine<DIM>(f, c, m[p], vol0[p], scale, dt, mu, lambda, out);
        wave_count(inverted, &status[0]);
        store_mat<DIM>(Cout, np, p, out);
    }
}

template <int DIM>
__global__ void __launch_bounds__(256) update_F_kernel(int64_t np, const float *__restrict__ C, float *__restrict__ F,
                                                       float dt)
{
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        float f[DIM][DIM], c[DIM][DIM];
        load_mat<DIM>(C, np, p, c);
        load_mat<DIM>(F, np, p, f);
        updated_F<DIM>(c, dt, f);
        store_mat<DIM>(F, np, p, f);
    }
}

// The two passes of one particle in one: F updated with the new C, then C'
// of the next substep from the updated F and the same C (C, F, m and vol0
// read once; F and C' written).
template <int DIM>
__global__ void __launch_bounds__(256) update_F_stress_kernel(int64_t np, double scale, const float *__restrict__ C,
                                                              float *__restrict__ F, const float *__restrict__ m,
                                                              const float *__restrict__ vol0, float dt, float mu,
                                                              float lambda, float *__restrict__ Cout,
                                                              uint32_t *__restrict__ status)
{
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        float f[DIM][DIM], c[DIM][DIM], out[DIM][DIM];
        load_mat<DIM>(C, np, p, c);
        load_mat<DIM>(F, np, p, f);
        updated_F<DIM>(c, dt, f);
        store_mat<DIM>(F, np, p, f);
        const bool inverted = stressed_affine<DIM>(f, c, m[p], vol0[p], scale, dt, mu, lambda, out);
        wave_count(inverted, &status[0]);
        store_mat<DIM>(Cout, np, p, out);
    }
}

// One thread per particle (measured faster than a grid of 16 blocks per CU
// striding over several: 0.246 against 0.266 ms for the F update with stress
// on 8M particles).
int stress_blocks(int64_t np)
{
    const int64_t want = (np + 255) / 256;
    return (int)(want < 1 ? 1 : want);
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

hipError_t launch_update_F_stress(int dim, int n, int64_t np, const float *C, float *F, const float *m,
                                  const float *vol0, float dt, float mu, float lambda, float *Cout, uint32_t *status,
                                  hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const double scale = 4.0 * (double)n * (double)n;
    if (dim == 3)
        hipLaunchKernelGGL(update_F_stress_kernel<3>, dim3(stress_blocks(np)), dim3(256), 0, s, np, scale, C, F, m,
                           vol0, dt, mu, lambda, Cout, status);
    else
        hipLaunchKernelGGL(update_F_stress_kernel<2>, dim3(stress_blocks(np)), dim3(256), 0, s, np, scale, C, F, m,
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
