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

// Quotients a / b of several numerators over one positive denominator b,
// each bit-identical to the correctly rounded float64 division that the
// compiler emits for a / b.  That division scales both operands when their
// exponents are extreme, takes the hardware reciprocal of the (scaled)
// denominator and refines it with two Newton steps, multiplies the numerator
// by it, corrects the product once with its exact FMA residual, and fixes up
// special values.  Inside the range that div_safe accepts no scaling and no
// fix-up happens (no operand, reciprocal or quotient is denormal, zero,
// infinite or near overflow, and the exponents differ by far less than the
// 768 at which the denominator is scaled), so the reciprocal and its two
// refinements depend on b alone and are formed once for all numerators; each
// quotient then costs a multiply and two FMAs instead of the whole sequence.
// The final correction is written as -fma(-e, r, -q), the same rounding as
// fma(e, r, q), so that a -0 numerator gives -0 as the division does.
__device__ __forceinline__ double recip_refined(double b)
{
    double r = __builtin_amdgcn_rcp(b);
    double t = __builtin_fma(-b, r, 1.0);
    r = __builtin_fma(r, t, r);
    t = __builtin_fma(-b, r, 1.0);
    return __builtin_fma(r, t, r);
}

__device__ __forceinline__ double div_refined(double a, double b, double rb)
{
    const double q = a * rb;
    const double e = __builtin_fma(-b, q, a);
    return -__builtin_fma(-e, rb, -q);
}

// The operands for which div_refined equals a / b: a denominator in
// [2^-100, 2^100] and numerators that are zero or in [2^-700, 2^200] in
// magnitude (quotients then in [2^-800, 2^300]).
// (Bitwise, not short-circuit, operators: the tests are compares, not branches.)
__device__ __forceinline__ bool div_denominator_safe(double b) { return (b >= 0x1p-100) & (b <= 0x1p100); }
__device__ __forceinline__ bool div_numerator_safe(double a)
{
    const double m = fabs(a);
    return (a == 0.0) | ((m >= 0x1p-700) & (m <= 0x1p200));
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
// non-positive determinant.  The divisions by det R and det F run through
// div_refined where div_safe allows (the same bits as the division).
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
    // A lane whose iterate turns singular stops updating R (and returns
    // false); the loop has no early exit, so R needs no copy per step.
    for (int k = 0; k < polar_iters; ++k) {
        if (ok) {
            const double det = pbmpm_cofactor<DIM>(r, cof);
            const double det2 = det + det;               // exact
            bool fast = div_denominator_safe(det2);
#pragma unroll
            for (int d = 0; d < DIM; ++d)
#pragma unroll
                for (int e = 0; e < DIM; ++e)
                    fast = fast & div_numerator_safe(cof[d][e]);
            if (!(det > 0.0)) {
                ok = false;
            } else if (fast) {
                // RN(RN(R + q) / 2) with q = RN(cof / det) is RN(R / 2 +
                // RN(cof / (2 det))), one FMA: halving commutes with rounding
                // in the normal range, and here q/2 is 0 or at least 2^-801 in
                // magnitude, so neither side rounds into the subnormals.
                const double rdet2 = recip_refined(det2);
#pragma unroll
                for (int d = 0; d < DIM; ++d)
#pragma unroll
                    for (int e = 0; e < DIM; ++e)
                        r[d][e] = __builtin_fma(r[d][e], 0.5, div_refined(cof[d][e], det2, rdet2));
            } else {
#pragma unroll
                for (int d = 0; d < DIM; ++d)
#pragma unroll
                    for (int e = 0; e < DIM; ++e)
                        r[d][e] = (r[d][e] + cof[d][e] / det) * 0.5;
            }
        }
    }
    const double detf = ok ? pbmpm_cofactor<DIM>(f, cof) : 0.0;
    if (!ok || !(detf > 0.0))
        return false;
    double finv[3][3];
    bool fast = div_denominator_safe(detf);
#pragma unroll
    for (int q = 0; q < DIM; ++q)
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            fast = fast & div_numerator_safe(cof[e][q]);
    if (fast) {
        const double rdet = recip_refined(detf);
#pragma unroll
        for (int q = 0; q < DIM; ++q)
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                finv[q][e] = div_refined(cof[e][q], detf, rdet);
    } else {
#pragma unroll
        for (int q = 0; q < DIM; ++q)
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                finv[q][e] = cof[e][q] / detf;
    }
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

// particleIntegrate for one particle, without the deformation update:
// x_e <- x_e + d_e (float32) clamped to [lo, hi] = [dx, (n - 2) dx]; then
// d_e <- d_e + gdt2_e (gravity into the next substep's displacement, gdt2_e =
// g_e * (dt * dt) formed once on the host in float32).  Returns whether a
// coordinate was clamped.
template <int DIM>
__device__ __forceinline__ bool pbmpm_integrate_particle(int64_t p, int64_t np, float *__restrict__ x,
                                                         float *__restrict__ d, float lo, float hi,
                                                         const float (&gdt2)[3])
{
    bool clamped = false;
#pragma unroll
    for (int e = 0; e < DIM; ++e) {
        const float de = d[(int64_t)e * np + p];
        const float xa = x[(int64_t)e * np + p] + de;
        const float xc = fminf(fmaxf(xa, lo), hi);
        clamped = clamped || xc != xa;
        x[(int64_t)e * np + p] = xc;
        d[(int64_t)e * np + p] = de + gdt2[e];
    }
    return clamped;
}

// The G2P gather with dt = 0 (d and D from the displacement grid dg, x kept)
// followed by the projection above, one pass (grid.hip).
// bins: a checked binning of these particles whose records the gather
// rewrites from the new state (with the binning's ranges r and the masses m),
// or NULL.
// The loop's last G2P gather (dt = 0), then per particle the integrate step
// and F <- (I + D) F, one launch (grid.hip).
hipError_t launch_pbmpm_g2p_integrate(int dim, int n, const float *dg, float *x, float *d, float *D, int64_t np,
                                      float *F, float dt, const float *gravity, uint32_t *status, hipStream_t s);

hipError_t launch_pbmpm_g2p_project(int dim, int n, const float *dg, float *x, float *d, float *D, int64_t np,
                                    const float *F, float relax, int polar_iters, uint32_t *status, hipStream_t s,
                                    const BinView *bins = nullptr, RangesF r = RangesF{}, const float *m = nullptr);

}  // namespace mpmk
