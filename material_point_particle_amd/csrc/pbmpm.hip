// pbmpm.hip -- the per-particle steps of the position-based MPM (PB-MPM)
// iteration loop for an elastic material ("Implementation -- GPU
// Optimization & Reference Codebases", section 3.3.2).
//
// A particle carries its displacement over the substep d (in the velocity
// array) and its displacement gradient D (in the affine-matrix array, same
// layout), with x, m and the deformation gradient F.  A substep is
// `iterations` times { the elastic projection of D (this file), binning and
// P2G of m and m (d + D (x_i - x_p)) (the APIC P2G with v := d, C := D; no
// stress term), the displacement-form grid update (grid.hip, node_rows_kernel
// OP 2) and the G2P gather of d and D (the G2P kernel with dt = 0, which
// leaves x in place) }, then the integrate step (this file) and
// F <- (I + D) F (stress.hip's F update with dt = 1).  The per-particle
// projection lives in pbmpm_device.hpp, so that grid.hip's gather can run the
// next iteration's projection in the same pass.
#include "pbmpm_device.hpp"

namespace mpmk {
namespace {

// particleUpdate for an elastic material (pbmpm_project_particle): a
// particle whose Ft or F (or a Newton iterate) has a non-positive determinant
// keeps D and is counted in status[0].  One thread per particle.
template <int DIM>
__global__ void __launch_bounds__(256) pbmpm_project_kernel(int64_t np, const float *__restrict__ F,
                                                            float *__restrict__ D, double relax, int polar_iters,
                                                            uint32_t *__restrict__ status)
{
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x) {
        float ds[DIM * DIM];
#pragma unroll
        for (int q = 0; q < DIM * DIM; ++q)
            ds[q] = D[(int64_t)q * np + p];
        const bool ok = pbmpm_project_particle<DIM>(
            [&](int q) { return F[(int64_t)q * np + p]; }, ds, relax, polar_iters,
            [&](int q, float val) { D[(int64_t)q * np + p] = val; });
        wave_count(!ok, &status[0]);
    }
}

// particleIntegrate for an elastic material, without the deformation update
// (pbmpm_integrate_particle); clamped particles counted in status[2].
template <int DIM>
__global__ void __launch_bounds__(256) pbmpm_integrate_kernel(int64_t np, float *__restrict__ x,
                                                              float *__restrict__ d, float lo, float hi, float gx,
                                                              float gy, float gz, uint32_t *__restrict__ status)
{
    const float gdt2[3] = { gx, gy, gz };
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < np; p += (int64_t)gridDim.x * blockDim.x)
        wave_count(pbmpm_integrate_particle<DIM>(p, np, x, d, lo, hi, gdt2), &status[2]);
}

// One thread per particle (the per-particle passes here measured no slower,
// and the integrate step faster, than with a capped grid striding over
// several).
int blocks_for(int64_t work, int block)
{
    const int64_t want = (work + block - 1) / block;
    return (int)(want < 1 ? 1 : want);
}

}  // namespace

hipError_t launch_pbmpm_project(int dim, int64_t np, const float *F, float *D, float relax, int polar_iters,
                                uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    if (dim == 3)
        hipLaunchKernelGGL(pbmpm_project_kernel<3>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, F, D,
                           (double)relax, polar_iters, status);
    else
        hipLaunchKernelGGL(pbmpm_project_kernel<2>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, F, D,
                           (double)relax, polar_iters, status);
    return hipGetLastError();
}

hipError_t launch_pbmpm_integrate(int dim, int n, int64_t np, float *x, float *d, float dt, const float *gravity,
                                  uint32_t *status, hipStream_t s)
{
    if (np == 0)
        return hipSuccess;
    const float dx = 1.0f / (float)n;
    float gdt2[3] = { 0.0f, 0.0f, 0.0f };
    for (int e = 0; e < dim; ++e)
        gdt2[e] = gravity[e] * (dt * dt);
    if (dim == 3)
        hipLaunchKernelGGL(pbmpm_integrate_kernel<3>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, x, d, dx,
                           (float)(n - 2) * dx, gdt2[0], gdt2[1], gdt2[2], status);
    else
        hipLaunchKernelGGL(pbmpm_integrate_kernel<2>, dim3(blocks_for(np, 256)), dim3(256), 0, s, np, x, d, dx,
                           (float)(n - 2) * dx, gdt2[0], gdt2[1], gdt2[2], status);
    return hipGetLastError();
}

}  // namespace mpmk
