// pbmpm_device.hpp -- the elastic particleUpdate of the position-based MPM
// loop for one particle ("Implementation -- GPU Optimization & Reference
// Codebases", section 3.3.2), shared by the projection kernel (pbmpm.hip) and
// the G2P gather that runs the next iteration's projection in the same pass
// (grid.hip), so both compute the same bits.
#pragma once
#include "common.hpp"

namespace mpmk {

// Cofactor matrix of the dim x dim matrix a (a^-T = cof / det); returns
// det a = (a00 cof00 + a01 cof01) + a02 cof02 (2D: a00 a11 - a01 a10).
template <int DIM>
__device__ __forceinline__ double pbmpm_cofactor(const double (&a)[3][3], double (&cof)[3][3])
{
    if constexpr (DIM == 3) {
        cof[0][0] = a[1][1] * a[2][2] - a[1][2] * a[2][1];
        cof[0][1] = a[1][2] * a[2][0] - a[1][0] * a[2][2];
        cof[0][2] = a[1][0] * a[2][1] - a[1][1] * a[2][0];
        cof[1][0] = a[0][2] * a[2][1] - a[0][1] * a[2][2];
        cof[1][1] = a[0][0] * a[2][2] - a[0][2] * a[2][0];
        cof[1][2] = a[0][1] * a[2][0] - a[0][0] * a[2][1];
        cof[2][0] = a[0][1] * a[1][2] - a[0][2] * a[1][1];
        cof[2][1] = a[0][2] * a[1][0] - a[0][0] * a[1][2];
        cof[2][2] = a[0][0] * a[1][1] - a[0][1] * a[1][0];
        return (a[0][0] * cof[0][0] + a[0][1] * cof[0][1]) + a[0][2] * cof[0][2];
    } else {
        cof[0][0] = a[1][1];
        cof[0][1] = -a[1][0];
        cof[1][0] = -a[0][1];
        cof[1][1] = a[0][0];
        return a[0][0] * a[1][1] - a[0][1] * a[1][0];
    }
}

// particleUpdate for an elastic material: the target shape is the polar
// rotation R of the trial deformation Ft = (I + D) F (Newton's iteration
// R <- (R + R^-T) / 2 from R = Ft, polar_iters steps); the displacement
// gradient reaching it is D* = R F^-1 - I; D <- D + relax (D* - D).  Float64
// in this order, D rounded to float32 once:
//   Ft_de = sum_q ([d == q] + D_dq) F_qe                  (q ascending)
//   R_de <- (R_de + cof(R)_de / det R) * 0.5
//   F^-1_qe = cof(F)_eq / det F
//   D*_de = (sum_q R_dq F^-1_qe) - [d == e]
//   D_de <- D_de + relax * (D*_de - D_de)
// loadF(q) gives F's entry q and D holds D, row-major (entry (d, e) at
// q = d * DIM + e); the new D goes out through store(q, value), entry by
// entry as it is formed (so that no second copy of it stays live).  Returns
// false, with nothing stored, when Ft, F or a Newton iterate has a
// non-positive determinant.
template <int DIM, class LoadF, class Store>
__device__ __forceinline__ bool pbmpm_project_particle(LoadF &&loadF, const float (&D)[DIM * DIM], double relax,
                                                       int polar_iters, Store &&store)
{
    double f[3][3] = {}, dd[3][3] = {}, ft[3][3] = {}, r[3][3] = {}, cof[3][3] = {};
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            f[d][e] = (double)loadF(d * DIM + e);
            dd[d][e] = (double)D[d * DIM + e];
        }
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            double t = ((d == 0 ? 1.0 : 0.0) + dd[d][0]) * f[0][e];
#pragma unroll
            for (int q = 1; q < DIM; ++q)
                t = t + ((d == q ? 1.0 : 0.0) + dd[d][q]) * f[q][e];
            ft[d][e] = t;
            r[d][e] = t;
        }
    bool ok = pbmpm_cofactor<DIM>(ft, cof) > 0.0;
    for (int k = 0; k < polar_iters; ++k) {
        if (!ok)
            break;
        const double det = pbmpm_cofactor<DIM>(r, cof);
        if (!(det > 0.0)) {
            ok = false;
            break;
        }
#pragma unroll
        for (int d = 0; d < DIM; ++d)
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                r[d][e] = (r[d][e] + cof[d][e] / det) * 0.5;
    }
    const double detf = ok ? pbmpm_cofactor<DIM>(f, cof) : 0.0;
    if (!ok || !(detf > 0.0))
        return false;
    double finv[3][3];
#pragma unroll
    for (int q = 0; q < DIM; ++q)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            finv[q][e] = cof[e][q] / detf;
#pragma unroll
    for (int d = 0; d < DIM; ++d)
#pragma unroll
        for (int e = 0; e < DIM; ++e) {
            double t = r[d][0] * finv[0][e];
#pragma unroll
            for (int q = 1; q < DIM; ++q)
                t = t + r[d][q] * finv[q][e];
            const double dstar = t - (d == e ? 1.0 : 0.0);
            store(d * DIM + e, (float)(dd[d][e] + relax * (dstar - dd[d][e])));
        }
    return true;
}

// The G2P gather with dt = 0 (d and D from the displacement grid dg, x kept)
// followed by the projection above, one pass (grid.hip).
// bins: a checked binning of these particles whose records the gather
// rewrites from the new state (with the binning's ranges r and the masses m),
// or NULL.
hipError_t launch_pbmpm_g2p_project(int dim, int n, const float *dg, float *x, float *d, float *D, int64_t np,
                                    const float *F, float relax, int polar_iters, uint32_t *status, hipStream_t s,
                                    const BinView *bins = nullptr, RangesF r = RangesF{}, const float *m = nullptr);

}  // namespace mpmk
