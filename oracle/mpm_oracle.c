/*
 * mpm_oracle.c -- plain, slow, single-threaded CPU oracle for the material
 * point method's particle-to-grid (P2G) transfer and the three steps around it
 * (binning, grid update, grid-to-particle).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call,
 * link or load this file; only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library: the two are written separately from the same definitions.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no -ffast-math,
 * no -march=native), so every float operation is one IEEE binary32 operation
 * rounded to nearest even, in the order written below.  OpenMP is used only
 * by oracle_p2g_quadratic_threads (the CPU baseline's all-cores leg); every
 * other function is single-threaded.
 *
 * Sources (pages as titled):
 *  - "particle to grid transfer in checked integer arithmetic" (integerc.dev),
 *    sections "integers do not care about order" and "the program": the
 *    integer split of a quantity between near and far nodes, done along x and
 *    then along y, and the bounds line run before any scatter; section "what
 *    is not claimed": quadratic weights and the affine term as further splits
 *    of the same kind (the integer-split quadratic APIC transfer below).
 *  - "Implementation -- GPU Optimization & Reference Codebases" (vocaro.com),
 *    section 1 (the four-phase step reset -> P2G -> grid update -> G2P),
 *    section 2.1 (fixed-point accumulation, tiles), section 3.1 (APIC
 *    transfer with the 3x3 quadratic B-spline stencil and affine matrix C;
 *    part 2 of the guide described there: the Neo-Hookean stress and the
 *    deformation gradient),
 *    section 3.3.1 (rounding, not truncating, fixed-point encode), section 5
 *    rules 1, 4, 7 and 9 (integer accumulation converted once in the grid
 *    update; consume-and-zero; gravity owned by the solver; counted
 *    overflows).
 *  - "Mass Matrix Assembly on Tensor Cores for Implicit PIC" (arXiv
 *    2604.19286), section on shape functions: tensor-product B-splines,
 *    partition of unity, and the rule that places a second-order stencil on
 *    nodes {j-1, j, j+1} or {j, j+1, j+2} by whether the fractional
 *    coordinate is below one half.
 *  - "Particle worlds, part 3" (ericlevin.dev), steps 3 and 4: counting sort
 *    by cell as histogram, exclusive prefix sum and scatter.
 *
 * Readings taken where the pages leave a step open are listed with each
 * function.  The quadratic B-spline's formula is not legible on the pages
 * (the equation was lost in extraction); the textbook piecewise form is used:
 * N(t) = 3/4 - t^2 for |t| < 1/2, (3/2 - |t|)^2 / 2 for 1/2 <= |t| < 3/2,
 * else 0, which has the support and partition of unity the PIC page states.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status counters shared by every function that can skip work */
enum { ST_DOMAIN = 0, ST_RANGE = 1, ST_CLAMP = 2 };

/* ------------------------------------------------------------------------ */
/* Integer split cloud-in-cell (integer-arithmetic page).                    */
/* ------------------------------------------------------------------------ */

/* t / 65536 rounded to the nearest integer, ties to the even neighbour,
 * computed in integers only.  (The page says "rounded once to the nearest
 * integer" without a tie rule; ties to even is the reading taken.) */
static int64_t div65536_nearest_even(int64_t t)
{
    int64_t fl = t / 65536;
    if (t % 65536 != 0 && t < 0)
        fl -= 1;                            /* floor division */
    int64_t r = t - fl * 65536;             /* 0 <= r < 65536 */
    if (r > 32768)
        return fl + 1;
    if (r == 32768)
        return fl + (fl & 1);
    return fl;
}

/* The far node's share of q at fraction f/65536 toward it. */
int64_t oracle_split_far(int64_t q, int32_t f)
{
    return div65536_nearest_even(q * (int64_t)f);
}

/* Bounds line: particle count x largest mass x largest speed, and the largest
 * product q * f formed by a split, must fit a signed 64-bit integer.
 * Returns 1 when the scatter may run, 0 when it must stop before any work. */
int oracle_cic_bounds_ok(int64_t n, int64_t max_mass, int64_t max_speed)
{
    long double node_bound = (long double)n * (long double)max_mass * (long double)(max_speed > 1 ? max_speed : 1);
    long double split_bound = (long double)max_mass * (long double)(max_speed > 1 ? max_speed : 1) * 65536.0L;
    long double lim = 9223372036854775807.0L;
    return node_bound <= lim && split_bound <= lim;
}

/*
 * Scatter n particles (in `order`, or index order when order is NULL) onto a
 * (cells+1) x (cells+1) node grid.  Positions X[2][n] are in units of 1/65536
 * of a cell; masses m[n] and velocities vel[2][n] are integers.  The three
 * quantities q = m, m*vx, m*vy are each split along x between the near node
 * (cell index) and the far node (index + 1), and each x part is then split
 * along y the same way.  grid[3][cells+1][cells+1] (x fastest) is
 * accumulated into.  Particles outside [0, cells) are skipped and counted in
 * status[0].
 */
void oracle_p2g_cic_split(int64_t n, const int32_t *X, const int32_t *m, const int32_t *vel,
                          const int64_t *order, int32_t cells, int64_t *grid, uint32_t *status)
{
    const int64_t nn = (int64_t)(cells + 1);
    const int64_t span = (int64_t)cells * 65536;
    for (int64_t k = 0; k < n; ++k) {
        int64_t p = order ? order[k] : k;
        int64_t px = X[p], py = X[n + p];
        if (px < 0 || px >= span || py < 0 || py >= span) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        int64_t cx = px / 65536, cy = py / 65536;
        int32_t fx = (int32_t)(px % 65536), fy = (int32_t)(py % 65536);
        int64_t q[3];
        q[0] = m[p];
        q[1] = (int64_t)m[p] * vel[p];
        q[2] = (int64_t)m[p] * vel[n + p];
        for (int c = 0; c < 3; ++c) {
            int64_t far_x = oracle_split_far(q[c], fx);
            int64_t near_x = q[c] - far_x;
            int64_t part[2] = { near_x, far_x };
            for (int i = 0; i < 2; ++i) {
                int64_t far_y = oracle_split_far(part[i], fy);
                int64_t near_y = part[i] - far_y;
                grid[(c * nn + (cy + 0)) * nn + (cx + i)] += near_y;
                grid[(c * nn + (cy + 1)) * nn + (cx + i)] += far_y;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Integer-split quadratic APIC transfer.                                    */
/* ------------------------------------------------------------------------ */

/*
 * The integer page's split carried to the quadratic B-spline and the affine
 * term (its "what is not claimed" section: both would be more splits of the
 * same kind; reading 18).  Positions are integers in units of 2^-16 cell; along
 * one axis the base node is floor(g - 1/2) and F = X - 2^16 base is the
 * distance from it, in [2^15, 3 2^15).  The quadratic B-spline weights are
 * then exact dyadic rationals over 2^33:
 *   W0 = (3 2^15 - F)^2,  W2 = (F - 2^15)^2,  W1 = 2^33 - W0 - W2.
 * A quantity q is split over the three nodes by rounding the two outer shares
 * (nearest, ties even) and giving the middle node the rest, so the shares sum
 * to q exactly.  The affine term needs the first-moment weights
 * u_o = w_o (o - f), which sum to zero: U0 = -W0 F and U2 = W2 (2^17 - F) over
 * 2^49, the outer shares rounded, the middle share minus their sum, so the
 * shares sum to exactly zero.
 */

/* t / 2^k rounded to nearest, ties to the even neighbour (128-bit t). */
static int64_t rhe_shift128(__int128 t, int k)
{
    __int128 fl = t >> k;                       /* arithmetic shift: floor */
    __int128 r = t - fl * ((__int128)1 << k);   /* 0 <= r < 2^k */
    __int128 half = (__int128)1 << (k - 1);
    if (r > half || (r == half && (fl & 1) != 0))
        fl += 1;
    return (int64_t)fl;
}

/* kind 0: the weights w; kind 1: the first-moment weights u. */
static void split_1d(int64_t q, int64_t F, int kind, int64_t s[3])
{
    const __int128 W0 = (__int128)(3 * 32768 - F) * (3 * 32768 - F);
    const __int128 W2 = (__int128)(F - 32768) * (F - 32768);
    if (kind == 0) {
        s[0] = rhe_shift128((__int128)q * W0, 33);
        s[2] = rhe_shift128((__int128)q * W2, 33);
        s[1] = q - s[0] - s[2];
    } else {
        s[0] = rhe_shift128((__int128)q * (-W0 * F), 49);
        s[2] = rhe_shift128((__int128)q * (W2 * (131072 - F)), 49);
        s[1] = -s[0] - s[2];
    }
}

/* Tensor split of q over the 3^dim stencil: along x, then each x share along
 * y, then each of those along z; kinds[e] picks w or u on axis e.  out is
 * indexed [a][b][c] as out[(a * 3 + b) * 3 + c] (2D: c = 0). */
static void split_tensor(int dim, int64_t q, const int64_t F[3], const int kinds[3], int64_t out[27])
{
    int64_t sx[3];
    split_1d(q, F[0], kinds[0], sx);
    for (int a = 0; a < 3; ++a) {
        int64_t sy[3];
        split_1d(sx[a], F[1], kinds[1], sy);
        for (int b = 0; b < 3; ++b) {
            if (dim == 3) {
                int64_t sz[3];
                split_1d(sy[b], F[2], kinds[2], sz);
                for (int c = 0; c < 3; ++c)
                    out[(a * 3 + b) * 3 + c] = sz[c];
            } else {
                out[(a * 3 + b) * 3] = sy[b];
            }
        }
    }
}

/*
 * Scatter np particles (in `order`, or index order) onto the int64 grid
 * [1+dim][n]^dim (x fastest).  X[dim][np]: positions in 2^-16 cell; m[np],
 * v[dim][np], C[dim*dim][np]: integers, C_de in velocity per cell, so that a
 * particle's exact contribution to node i is m w_i (v + C (i - g)) with the
 * offset in cells.  Mass: the tensor split of m.  Momentum d: the tensor split
 * of m v_d, plus for every axis e the tensor split of m C_de with the
 * first-moment weights on axis e (and the weights on the others).  Node totals
 * equal particle totals exactly: sum M = sum m, sum P_d = sum m v_d.
 * Particles whose stencil leaves the grid are skipped and counted in
 * status[0].
 */
void oracle_p2g_isplit(int dim, int n, int64_t np_, const int32_t *X, const int64_t *m, const int64_t *v,
                       const int64_t *C, const int64_t *order, int64_t *grid, uint32_t *status)
{
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const int nc = dim == 3 ? 3 : 1;
    for (int64_t k = 0; k < np_; ++k) {
        const int64_t p = order ? order[k] : k;
        int64_t base[3] = { 0, 0, 0 }, F[3] = { 65536, 65536, 65536 };
        int ok = 1;
        for (int e = 0; e < dim; ++e) {
            const int64_t x = X[e * np_ + p];
            int64_t t = x - 32768, b = t / 65536;
            if (t % 65536 != 0 && t < 0)
                b -= 1;                                 /* floor */
            base[e] = b;
            F[e] = x - b * 65536;
            ok &= b >= 0 && b <= n - 3;
        }
        if (!ok) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        int64_t share[1 + 3][27];
        memset(share, 0, sizeof(share));
        const int w_only[3] = { 0, 0, 0 };
        split_tensor(dim, m[p], F, w_only, share[0]);
        for (int d = 0; d < dim; ++d) {
            int64_t part[27];
            split_tensor(dim, m[p] * v[d * np_ + p], F, w_only, part);
            for (int i = 0; i < 27; ++i)
                share[1 + d][i] += part[i];
            for (int e = 0; e < dim; ++e) {
                int kinds[3] = { 0, 0, 0 };
                kinds[e] = 1;
                split_tensor(dim, m[p] * C[(int64_t)(d * dim + e) * np_ + p], F, kinds, part);
                for (int i = 0; i < 27; ++i)
                    share[1 + d][i] += part[i];
            }
        }
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b)
                for (int c = 0; c < nc; ++c) {
                    const int64_t node = dim == 3
                        ? ((base[2] + c) * n + (base[1] + b)) * n + (base[0] + a)
                        : (base[1] + b) * n + (base[0] + a);
                    for (int ch = 0; ch <= dim; ++ch)
                        grid[ch * nodes + node] += share[ch][(a * 3 + b) * 3 + c];
                }
    }
}

/* Bounds line of the integer-split transfer: every split product fits the
 * 128-bit intermediate by construction; the node sums fit int64 when
 * np * max_mass * (max_speed + dim * max_affine * 3/2 + 1) < 2^62 (each share's
 * magnitude is at most its quantity's, plus the rounding).  1: may run. */
int oracle_isplit_bounds_ok(int dim, int64_t np_, int64_t max_mass, int64_t max_speed, int64_t max_affine)
{
    long double b = (long double)np_ * (long double)max_mass *
                    ((long double)max_speed + (long double)dim * (long double)max_affine * 1.5L + 1.0L);
    return b < 4611686018427387904.0L;
}

/* ------------------------------------------------------------------------ */
/* Quadratic B-spline APIC transfer.                                         */
/* ------------------------------------------------------------------------ */

/*
 * Stencil of one particle along one axis, with g = x * n in node units:
 * base = floor(g - 1/2) (the PIC page's placement rule: nodes {j-1, j, j+1}
 * when the fraction is below one half, else {j, j+1, j+2}); f = g - base in
 * [1/2, 3/2) is the distance from the base node; the three weights are the
 * quadratic B-spline at distances f, f-1, f-2; r[o] = (o - f) * dx is the
 * offset of node base+o from the particle in domain units.
 * Returns 0 when base falls outside [0, n-3] (the stencil would leave the
 * grid) or the coordinate is not finite.
 */
static int stencil_1d(float x, int n, int *base, float w[3], float r[3])
{
    float g = x * (float)n;
    float b = floorf(g - 0.5f);
    if (!(b >= 0.0f && b <= (float)(n - 3)))
        return 0;
    float f = g - b;
    float dx = 1.0f / (float)n;
    w[0] = 0.5f * ((1.5f - f) * (1.5f - f));
    w[1] = 0.75f - ((f - 1.0f) * (f - 1.0f));
    w[2] = 0.5f * ((f - 0.5f) * (f - 0.5f));
    for (int o = 0; o < 3; ++o)
        r[o] = ((float)o - f) * dx;
    *base = (int)b;
    return 1;
}

/* Is every attribute inside the declared ranges (the ranges the bounds check
 * proved safe)?  NaN fails every comparison and is therefore rejected. */
static int in_ranges(int dim, int64_t np_, int64_t p, const float *v, const float *C, const float *m,
                     double max_mass, double max_speed, double max_affine)
{
    if (!((double)fabsf(m[p]) <= max_mass))
        return 0;
    for (int d = 0; d < dim; ++d)
        if (!((double)fabsf(v[d * np_ + p]) <= max_speed))
            return 0;
    for (int k = 0; k < dim * dim; ++k)
        if (!((double)fabsf(C[k * np_ + p]) <= max_affine))
            return 0;
    return 1;
}

/*
 * Fixed-point APIC P2G with the quadratic B-spline stencil (3^dim nodes).
 *
 * Inputs (component-major): x[dim][np], v[dim][np], C[dim*dim][np] with
 * C[d*dim+e] the (row d, column e) entry of the affine matrix, m[np].
 * Output grid[(1+dim)][n^dim] (x fastest; channel 0 mass, channel 1+d
 * momentum d) is accumulated into.  S = 2^frac_bits.
 *
 * Per particle and node (a, b, c) of its stencil, all in float32:
 *   wmS = (((m * S) * wx[a]) * wy[b]) * wz[c]        (2D: no wz factor)
 *   u_d = ((v_d + C_d0 * rx[a]) + C_d1 * ry[b]) + C_d2 * rz[c]
 *   M   += (int64) rint(wmS)
 *   P_d += (int64) rint(wmS * u_d)
 * i.e. node mass m w and momentum m w (v + C (x_i - x_p)), scaled by S and
 * rounded to nearest (ties even) once per contribution.  The association
 * order above is this library's fixed reading (the pages fix no order); the
 * sums themselves are integer and so independent of particle order.
 *
 * Particles whose stencil leaves the grid are skipped and counted in
 * status[0]; particles outside the declared ranges are skipped and counted
 * in status[1] (domain is checked first).
 */
/* The particles at positions k0 .. k1-1 of the visiting order; touched (may
 * be NULL) gets a 1 for every 4^dim-node tile that receives a contribution. */
static void p2g_quadratic_range(int dim, int n, int frac_bits, int64_t np_, int64_t k0, int64_t k1,
                                const float *x, const float *v, const float *C, const float *m,
                                const int64_t *order, double max_mass, double max_speed, double max_affine,
                                int64_t *grid, uint32_t *status, uint8_t *touched)
{
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const int nt = n / 4;
    const float S = ldexpf(1.0f, frac_bits);
    for (int64_t k = k0; k < k1; ++k) {
        int64_t p = order ? order[k] : k;
        int base[3] = { 0, 0, 0 };
        float w[3][3] = { { 1, 0, 0 }, { 1, 0, 0 }, { 1, 0, 0 } };
        float r[3][3] = { { 0, 0, 0 }, { 0, 0, 0 }, { 0, 0, 0 } };
        int ok = 1;
        for (int e = 0; e < dim; ++e)
            ok &= stencil_1d(x[e * np_ + p], n, &base[e], w[e], r[e]);
        if (!ok) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        if (!in_ranges(dim, np_, p, v, C, m, max_mass, max_speed, max_affine)) {
            status[ST_RANGE] += 1;
            continue;
        }
        const float mS = m[p] * S;
        const int nc = dim == 3 ? 3 : 1;
        if (touched) {
            for (int tz = base[2] / 4; tz <= (dim == 3 ? (base[2] + 2) / 4 : 0); ++tz)
                for (int ty = base[1] / 4; ty <= (base[1] + 2) / 4; ++ty)
                    for (int tx = base[0] / 4; tx <= (base[0] + 2) / 4; ++tx)
                        touched[((int64_t)tz * nt + ty) * nt + tx] = 1;
        }
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b)
                for (int c = 0; c < nc; ++c) {
                    float wmS = (mS * w[0][a]) * w[1][b];
                    if (dim == 3)
                        wmS = wmS * w[2][c];
                    int64_t node = dim == 3
                        ? ((int64_t)(base[2] + c) * n + (base[1] + b)) * n + (base[0] + a)
                        : (int64_t)(base[1] + b) * n + (base[0] + a);
                    grid[node] += (int64_t)rintf(wmS);
                    for (int d = 0; d < dim; ++d) {
                        const float *Cd = C + (int64_t)d * dim * np_;
                        float u = (v[d * np_ + p] + Cd[0 * np_ + p] * r[0][a]) + Cd[1 * np_ + p] * r[1][b];
                        if (dim == 3)
                            u = u + Cd[2 * np_ + p] * r[2][c];
                        grid[(int64_t)(1 + d) * nodes + node] += (int64_t)rintf(wmS * u);
                    }
                }
    }
}

void oracle_p2g_quadratic(int dim, int n, int frac_bits, int64_t np_,
                          const float *x, const float *v, const float *C, const float *m,
                          const int64_t *order, double max_mass, double max_speed, double max_affine,
                          int64_t *grid, uint32_t *status)
{
    p2g_quadratic_range(dim, n, frac_bits, np_, 0, np_, x, v, C, m, order, max_mass, max_speed, max_affine, grid,
                        status, NULL);
}

/*
 * The same transfer on several host threads, for the CPU baseline's
 * all-cores measurement (not used by any test as a reference: the tests
 * compare it with oracle_p2g_quadratic).  The visiting order is cut into
 * nthreads contiguous ranges; each thread accumulates its range into a
 * private zeroed int64 grid with the arithmetic above and flags the 4^dim-node
 * tiles it wrote; then the private grids of every flagged tile are added into
 * `grid`, tile by tile in parallel.  Integer additions commute, so the result
 * is bit-identical to oracle_p2g_quadratic.  Returns 0, or -1 when the private
 * grids cannot be allocated (nothing is added then).
 */
int oracle_p2g_quadratic_threads(int dim, int n, int frac_bits, int64_t np_,
                                 const float *x, const float *v, const float *C, const float *m,
                                 const int64_t *order, double max_mass, double max_speed, double max_affine,
                                 int64_t *grid, uint32_t *status, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const int nt = n / 4;
    const int64_t tiles = dim == 3 ? (int64_t)nt * nt * nt : (int64_t)nt * nt;
    const int64_t words = (int64_t)(1 + dim) * nodes;
    int64_t **priv = calloc((size_t)nthreads, sizeof(int64_t *));
    uint8_t **flag = calloc((size_t)nthreads, sizeof(uint8_t *));
    uint32_t *st = calloc((size_t)nthreads * 4, sizeof(uint32_t));
    int ok = priv && flag && st;
    for (int t = 0; ok && t < nthreads; ++t) {
        priv[t] = calloc((size_t)words, sizeof(int64_t));
        flag[t] = calloc((size_t)tiles, 1);
        ok = priv[t] && flag[t];
    }
    if (ok) {
#pragma omp parallel for num_threads(nthreads) schedule(static, 1)
        for (int t = 0; t < nthreads; ++t) {
            const int64_t k0 = np_ * t / nthreads, k1 = np_ * (t + 1) / nthreads;
            p2g_quadratic_range(dim, n, frac_bits, np_, k0, k1, x, v, C, m, order, max_mass, max_speed, max_affine,
                                priv[t], st + 4 * t, flag[t]);
        }
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 64)
        for (int64_t tile = 0; tile < tiles; ++tile) {
            const int tx = (int)(tile % nt), ty = (int)((tile / nt) % nt), tz = dim == 3 ? (int)(tile / ((int64_t)nt * nt)) : 0;
            for (int t = 0; t < nthreads; ++t) {
                if (!flag[t][tile])
                    continue;
                for (int c = 0; c <= dim; ++c)
                    for (int z = 0; z < (dim == 3 ? 4 : 1); ++z)
                        for (int y = 0; y < 4; ++y)
                            for (int xx = 0; xx < 4; ++xx) {
                                const int64_t node = dim == 3
                                    ? ((int64_t)(tz * 4 + z) * n + (ty * 4 + y)) * n + (tx * 4 + xx)
                                    : (int64_t)(ty * 4 + y) * n + (tx * 4 + xx);
                                grid[(int64_t)c * nodes + node] += priv[t][(int64_t)c * nodes + node];
                            }
            }
        }
        for (int t = 0; t < nthreads; ++t)
            for (int i = 0; i < 4; ++i)
                status[i] += st[4 * t + i];
    }
    for (int t = 0; priv && flag && t < nthreads; ++t) {
        free(priv[t]);
        free(flag[t]);
    }
    free(priv);
    free(flag);
    free(st);
    return ok ? 0 : -1;
}

/*
 * Largest magnitude a single quantised contribution can take under the
 * declared ranges, in units of the fixed-point quantum:
 *   S * (3/4)^dim * max_mass * (max_speed + dim * max_affine * (3/2) dx)
 * (each 1D weight is at most 3/4 and each offset at most 3/2 cells), with a
 * small allowance for float32 rounding.  A P2G over np particles is safe in
 * int64 when np times this bound stays below 2^63.  Returns log2 of np times
 * the bound.
 */
double oracle_p2g_log2_bound(int dim, int n, int frac_bits, int64_t np_,
                             double max_mass, double max_speed, double max_affine)
{
    double dx = 1.0 / (double)n;
    double wmax = dim == 3 ? 0.421875 : 0.5625;
    double umax = max_speed + dim * max_affine * 1.5 * dx;
    if (umax < 1.0)
        umax = 1.0;   /* the mass channel has u = 1 */
    double q = ldexp(1.0, frac_bits) * wmax * max_mass * umax * (1.0 + 1e-6) + 1.0;
    return log2((double)(np_ > 0 ? np_ : 1) * q);
}

/* ------------------------------------------------------------------------ */
/* Grid update (consume-and-zero) and grid-to-particle gather.               */
/* ------------------------------------------------------------------------ */

/*
 * Per node: velocity v_d = P_d / M computed in double from the integer sums
 * and rounded once to float (zero where M == 0); where M != 0 the velocity
 * gains gravity, v_d = v_d + (dt * g_d) with dt * g_d formed once in float;
 * nodes within `sticky` nodes of any face get v = 0; finally the integer
 * accumulators are zeroed (each accumulator has exactly one reader, so the
 * clear rides along with the update).  vg[dim][n^dim] is written.
 */
void oracle_grid_update(int dim, int n, int64_t *grid, float *vg, float dt, const float *gravity, int sticky)
{
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    float gdt[3] = { 0, 0, 0 };
    for (int d = 0; d < dim; ++d)
        gdt[d] = dt * gravity[d];
    for (int64_t i = 0; i < nodes; ++i) {
        int64_t ix = i % n, iy = (i / n) % n, iz = dim == 3 ? i / ((int64_t)n * n) : 0;
        int64_t M = grid[i];
        float vel[3] = { 0, 0, 0 };
        if (M != 0) {
            for (int d = 0; d < dim; ++d) {
                vel[d] = (float)((double)grid[(1 + d) * nodes + i] / (double)M);
                vel[d] = vel[d] + gdt[d];
            }
        }
        int wall = ix < sticky || ix >= n - sticky || iy < sticky || iy >= n - sticky;
        if (dim == 3)
            wall = wall || iz < sticky || iz >= n - sticky;
        for (int d = 0; d < dim; ++d) {
            vg[d * nodes + i] = wall ? 0.0f : vel[d];
            grid[(1 + d) * nodes + i] = 0;
        }
        grid[i] = 0;
    }
}

/*
 * APIC gather: v = sum w vg and B = sum (w vg) r^T over the stencil (the
 * definition; the grouping below regroups these same sums exactly and only
 * fixes the float32 rounding order).  For each
 * particle, over its stencil nodes in lexicographic order (a outermost, then
 * b, then c), with w = (wx[a] * wy[b]) * wz[c]:
 *   wv_d        = w * vg_d(node)
 *   S[d][e][o] += wv_d     for each axis e, o the node's offset on axis e (from 0)
 * then vnew_d = (S[d][0][0] + S[d][0][1]) + S[d][0][2] and
 *   B_de = (r_e[0] * S[d][e][0] + r_e[1] * S[d][e][1]) + r_e[2] * S[d][e][2],
 * the same sums grouped by the offset along one axis (r_e depends on that
 * offset only); then C = B * (4 / dx^2) (the quadratic B-spline's inertia-like factor
 * dx^2/4 inverted), v = vnew, x_e = x_e + dt * v_e, and x_e is clamped to
 * [dx, (n-2) dx] (each clamped particle counted in status[2]).  Particles
 * whose stencil leaves the grid are left untouched and counted in status[0].
 */
void oracle_g2p(int dim, int n, const float *vg, int64_t np_, float *x, float *v, float *C, float dt,
                uint32_t *status)
{
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const float dx = 1.0f / (float)n;
    const float lo = dx, hi = (float)(n - 2) * dx;
    const float cscale = 4.0f * (float)n * (float)n;
    for (int64_t p = 0; p < np_; ++p) {
        int base[3] = { 0, 0, 0 };
        float w[3][3] = { { 1, 0, 0 }, { 1, 0, 0 }, { 1, 0, 0 } };
        float r[3][3] = { { 0, 0, 0 }, { 0, 0, 0 }, { 0, 0, 0 } };
        int ok = 1;
        for (int e = 0; e < dim; ++e)
            ok &= stencil_1d(x[e * np_ + p], n, &base[e], w[e], r[e]);
        if (!ok) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        /* S[d][e][o]: the sum of w * vg_d over the stencil nodes at offset o
         * along axis e, accumulated in lexicographic node order.  Since r_e
         * depends on the offset along axis e only, the sums over the stencil
         * v_d = sum w vg_d and B_de = sum (w vg_d) r_e are sum_o S[d][e][o] and
         * sum_o r_e[o] S[d][e][o]. */
        float S[3][3][3] = { { { 0 } } };
        float vnew[3] = { 0, 0, 0 };
        float B[3][3] = { { 0, 0, 0 }, { 0, 0, 0 }, { 0, 0, 0 } };
        const int nc = dim == 3 ? 3 : 1;
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b)
                for (int c = 0; c < nc; ++c) {
                    float wt = w[0][a] * w[1][b];
                    if (dim == 3)
                        wt = wt * w[2][c];
                    int64_t node = dim == 3
                        ? ((int64_t)(base[2] + c) * n + (base[1] + b)) * n + (base[0] + a)
                        : (int64_t)(base[1] + b) * n + (base[0] + a);
                    const int o[3] = { a, b, c };
                    for (int d = 0; d < dim; ++d) {
                        float wv = wt * vg[d * nodes + node];
                        for (int e = 0; e < dim; ++e)
                            S[d][e][o[e]] = S[d][e][o[e]] + wv;
                    }
                }
        for (int d = 0; d < dim; ++d) {
            vnew[d] = (S[d][0][0] + S[d][0][1]) + S[d][0][2];
            for (int e = 0; e < dim; ++e)
                B[d][e] = (r[e][0] * S[d][e][0] + r[e][1] * S[d][e][1]) + r[e][2] * S[d][e][2];
        }
        int clamped = 0;
        for (int d = 0; d < dim; ++d) {
            for (int e = 0; e < dim; ++e)
                C[(int64_t)(d * dim + e) * np_ + p] = B[d][e] * cscale;
            v[d * np_ + p] = vnew[d];
            float xn = x[d * np_ + p] + dt * vnew[d];
            float xc = fminf(fmaxf(xn, lo), hi);
            clamped |= xc != xn;
            x[d * np_ + p] = xc;
        }
        status[ST_CLAMP] += (uint32_t)clamped;
    }
}

/* ------------------------------------------------------------------------ */
/* MLS-MPM stress term of a Neo-Hookean solid.                               */
/* ------------------------------------------------------------------------ */

/*
 * "Implementation -- GPU Optimization & Reference Codebases", section 3.1,
 * part 2 of the guide: with J = det F and F^-T = (F^T)^-1,
 *   P = mu (F - F^-T) + lambda log(J) F^-T,   sigma = (1/J) P F^T.
 * In the MLS-MPM transfer the stress enters the affine term (reading 17): a
 * particle adds w_i (m v + Q (x_i - x_p)) to node i with
 * Q = m C - dt vol sigma D^-1, where D^-1 = 4 / dx^2 = 4 n^2 for the
 * quadratic B-spline (the inverse of sum_i w_i r_i r_i^T) and
 * vol sigma = vol0 J sigma = vol0 P F^T (vol0 the particle's initial volume).
 * Divided by m, the APIC P2G arithmetic is unchanged when its affine matrix is
 *   C' = C - k (P F^T),   k = dt vol0 4 n^2 / m.
 * Everything is float64 in the order written; each C' entry is rounded to
 * float32 once.  F^-T is the cofactor matrix over J.  Particles with
 * det F <= 0 (inverted) or m == 0 keep C' = C; the inverted ones are counted
 * in status[0].  F and C are component-major: entry (d, e) at [(d dim + e) np].
 */
void oracle_neohookean_affine(int dim, int n, int64_t np_, const float *F, const float *C, const float *m,
                              const float *vol0, float dt, float mu, float lambda, float *Cout, uint32_t *status)
{
    const double scale = 4.0 * (double)n * (double)n;
    for (int64_t p = 0; p < np_; ++p) {
        double f[3][3] = { { 0 } }, cof[3][3] = { { 0 } };
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                f[d][e] = (double)F[(int64_t)(d * dim + e) * np_ + p];
                Cout[(int64_t)(d * dim + e) * np_ + p] = C[(int64_t)(d * dim + e) * np_ + p];
            }
        double J;
        if (dim == 3) {
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
        if (!(J > 0.0)) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        if (m[p] == 0.0f)
            continue;
        const double llj = (double)lambda * log(J);
        double P[3][3];
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                const double fit = cof[d][e] / J;                       /* (F^-T)_de */
                P[d][e] = (double)mu * (f[d][e] - fit) + llj * fit;
            }
        const double k = (((double)dt * (double)vol0[p]) * scale) / (double)m[p];
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                double tau = 0.0;                                       /* (P F^T)_de */
                for (int q = 0; q < dim; ++q)
                    tau = tau + P[d][q] * f[e][q];
                const int64_t i = (int64_t)(d * dim + e) * np_ + p;
                Cout[i] = (float)((double)C[i] - k * tau);
            }
    }
}

/*
 * Deformation gradient update after G2P (the same part of the guide):
 * F <- (I + dt C) F with C the particle's new affine matrix, in float32:
 * G_dq = [d == q] + dt C_dq, then F'_de = sum_q G_dq F_qe in order q = 0, 1, 2.
 */
void oracle_update_F(int dim, int64_t np_, const float *C, float *F, float dt)
{
    for (int64_t p = 0; p < np_; ++p) {
        float G[3][3], f[3][3], out[3][3];
        for (int d = 0; d < dim; ++d)
            for (int q = 0; q < dim; ++q) {
                G[d][q] = (d == q ? 1.0f : 0.0f) + dt * C[(int64_t)(d * dim + q) * np_ + p];
                f[d][q] = F[(int64_t)(d * dim + q) * np_ + p];
            }
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                float t = G[d][0] * f[0][e];
                for (int q = 1; q < dim; ++q)
                    t = t + G[d][q] * f[q][e];
                out[d][e] = t;
            }
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e)
                F[(int64_t)(d * dim + e) * np_ + p] = out[d][e];
    }
}

/* ------------------------------------------------------------------------ */
/* Counting sort of particles by cell, cells numbered tile by tile.          */
/* ------------------------------------------------------------------------ */

/*
 * Cell key of a particle: its base cell (the stencil's base node, as in
 * stencil_1d) numbered tile-major: tiles of `tile` cells per axis in
 * row-major order, then the cells inside a tile in row-major order.
 * Returns -1 for a particle the transfer would skip (outside the domain or
 * the declared ranges).
 */
static int64_t cell_key(int dim, int n, int tile, int64_t np_, int64_t p, const float *x, const float *v,
                        const float *C, const float *m, double max_mass, double max_speed, double max_affine)
{
    int base[3] = { 0, 0, 0 };
    float w[3], r[3];
    for (int e = 0; e < dim; ++e)
        if (!stencil_1d(x[e * np_ + p], n, &base[e], w, r))
            return -1;
    if (!in_ranges(dim, np_, p, v, C, m, max_mass, max_speed, max_affine))
        return -1;
    int64_t nt = n / tile;
    int64_t t = 0, l = 0;
    for (int e = dim - 1; e >= 0; --e) {
        t = t * nt + base[e] / tile;
        l = l * tile + base[e] % tile;
    }
    int64_t per_tile = dim == 3 ? (int64_t)tile * tile * tile : (int64_t)tile * tile;
    return t * per_tile + l;
}

/*
 * Histogram of cell keys (cell_count[n_cells]), exclusive prefix sum
 * (cell_start[n_cells + 1]) and a stable scatter of particle indices into
 * order[] (particles the transfer would skip are left out).  Returns the
 * number of particles placed.  n_cells = n^dim.
 */
int64_t oracle_bin(int dim, int n, int tile, int64_t np_, const float *x, const float *v, const float *C,
                   const float *m, double max_mass, double max_speed, double max_affine,
                   uint32_t *cell_count, uint32_t *cell_start, int64_t *order)
{
    const int64_t n_cells = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(np_ > 0 ? np_ : 1));
    memset(cell_count, 0, sizeof(uint32_t) * (size_t)n_cells);
    for (int64_t p = 0; p < np_; ++p) {
        key[p] = cell_key(dim, n, tile, np_, p, x, v, C, m, max_mass, max_speed, max_affine);
        if (key[p] >= 0)
            cell_count[key[p]] += 1;
    }
    uint32_t run = 0;
    for (int64_t c = 0; c < n_cells; ++c) {
        cell_start[c] = run;
        run += cell_count[c];
    }
    cell_start[n_cells] = run;
    uint32_t *cursor = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n_cells);
    memcpy(cursor, cell_start, sizeof(uint32_t) * (size_t)n_cells);
    for (int64_t p = 0; p < np_; ++p)
        if (key[p] >= 0)
            order[cursor[key[p]]++] = p;
    free(cursor);
    free(key);
    return (int64_t)run;
}

/* ------------------------------------------------------------------------ */
/* Position-based MPM (PB-MPM), elastic material: the iteration loop of the  */
/* implementation page's section 3.3.2.                                      */
/* ------------------------------------------------------------------------ */
/*
 * A particle carries its displacement over the substep d (kept where the
 * APIC transfer keeps v) and its displacement gradient D (kept where it keeps
 * the affine matrix C, same layout), with x, m and the deformation gradient
 * F.  Per substep, `iterations` times:
 *   oracle_pbmpm_project_elastic   (particleUpdate: D toward the elastic target)
 *   oracle_p2g_quadratic           (particleToGrid of m and m (d + D (x_i - x_p)),
 *                                   with v := d and C := D; no stress term)
 *   oracle_pbmpm_grid_update       (gridUpdate in displacement form)
 *   oracle_g2p with dt = 0         (gridToParticle: gathers d and D = B 4 n^2;
 *                                   x stays in place)
 * then once: oracle_pbmpm_integrate (x += d, gravity into the next d) and
 * oracle_update_F with dt = 1 (F <- (I + D) F).  d and D persist into the next
 * substep (the warm start the page describes).
 */

/* Cofactor matrix of the dim x dim matrix a (so a^-T = cof / det); returns
 * det a = (a00 cof00 + a01 cof01) + a02 cof02 (2D: a00 a11 - a01 a10). */
static double pb_cofactor(int dim, const double a[3][3], double cof[3][3])
{
    if (dim == 3) {
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
    }
    cof[0][0] = a[1][1];
    cof[0][1] = -a[1][0];
    cof[1][0] = -a[0][1];
    cof[1][1] = a[0][0];
    return a[0][0] * a[1][1] - a[0][1] * a[1][0];
}

/*
 * particleUpdate for an elastic material.  The material's target shape is a
 * pure rotation: the polar rotation R of the trial deformation Ft = (I + D) F
 * (the U V^T of its SVD; the page replaces the SVD by Newton's polar
 * iteration in 3D: R <- (R + R^-T) / 2 from R = Ft, `polar_iters` steps).  The
 * displacement gradient that reaches the target is D* = R F^-1 - I, and D
 * relaxes toward it at rate `relax` (the page's elasticRelaxation, default 1.5,
 * over-relaxed): D <- D + relax (D* - D).  Everything in float64 in this order,
 * D rounded to float32 once:
 *   Ft_de = sum_q ([d == q] + D_dq) F_qe          (q ascending)
 *   R_de  <- (R_de + cof(R)_de / det R) * 0.5
 *   F^-1_qe = cof(F)_eq / det F
 *   D*_de = (sum_q R_dq F^-1_qe) - [d == e]
 *   D_de  <- D_de + relax * (D*_de - D_de)
 * A particle whose Ft or F has a non-positive determinant, or whose Newton
 * iterate loses it, keeps D and is counted in status[0].
 */
void oracle_pbmpm_project_elastic(int dim, int64_t np_, const float *F, float *D, float relax, int polar_iters,
                                  uint32_t *status)
{
    for (int64_t p = 0; p < np_; ++p) {
        double f[3][3] = { { 0 } }, dd[3][3] = { { 0 } }, ft[3][3] = { { 0 } }, r[3][3], cof[3][3];
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                f[d][e] = (double)F[(int64_t)(d * dim + e) * np_ + p];
                dd[d][e] = (double)D[(int64_t)(d * dim + e) * np_ + p];
            }
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                double t = ((d == 0 ? 1.0 : 0.0) + dd[d][0]) * f[0][e];
                for (int q = 1; q < dim; ++q)
                    t = t + ((d == q ? 1.0 : 0.0) + dd[d][q]) * f[q][e];
                ft[d][e] = t;
            }
        int ok = pb_cofactor(dim, ft, cof) > 0.0;
        for (int d = 0; d < 3; ++d)
            for (int e = 0; e < 3; ++e)
                r[d][e] = ft[d][e];
        for (int k = 0; ok && k < polar_iters; ++k) {
            const double det = pb_cofactor(dim, r, cof);
            if (!(det > 0.0)) {
                ok = 0;
                break;
            }
            for (int d = 0; d < dim; ++d)
                for (int e = 0; e < dim; ++e)
                    r[d][e] = (r[d][e] + cof[d][e] / det) * 0.5;
        }
        const double detf = ok ? pb_cofactor(dim, f, cof) : 0.0;
        if (!ok || !(detf > 0.0)) {
            status[ST_DOMAIN] += 1;
            continue;
        }
        double finv[3][3];
        for (int q = 0; q < dim; ++q)
            for (int e = 0; e < dim; ++e)
                finv[q][e] = cof[e][q] / detf;
        for (int d = 0; d < dim; ++d)
            for (int e = 0; e < dim; ++e) {
                double t = r[d][0] * finv[0][e];
                for (int q = 1; q < dim; ++q)
                    t = t + r[d][q] * finv[q][e];
                const double dstar = t - (d == e ? 1.0 : 0.0);
                const int64_t i = (int64_t)(d * dim + e) * np_ + p;
                D[i] = (float)(dd[d][e] + (double)relax * (dstar - dd[d][e]));
            }
    }
}

/*
 * gridUpdate in displacement form (section 3.3.2: mass-normalise, then the
 * guardian projects each node's displaced position back into bounds).  Per
 * node: where M != 0, d_e = (float)((double)P_e / (double)M), then with the
 * node's position X_e = i_e dx (exact in float32 for a power-of-two n),
 * d_e = fminf(fmaxf(X_e + d_e, lo), hi) - X_e with lo = band dx and
 * hi = (n - 1 - band) dx (float32, in this order); d = 0 where M == 0; then
 * M and P are set to 0 (consume-and-zero, as the velocity-form update).
 * No gravity here: the integrate step puts it into the next displacement.
 */
void oracle_pbmpm_grid_update(int dim, int n, int64_t *grid, float *dg, int band)
{
    const int64_t nodes = dim == 3 ? (int64_t)n * n * n : (int64_t)n * n;
    const float dx = 1.0f / (float)n;
    const float lo = (float)band * dx, hi = (float)(n - 1 - band) * dx;
    for (int64_t node = 0; node < nodes; ++node) {
        const int64_t M = grid[node];
        const int idx[3] = { (int)(node % n), (int)((node / n) % n), dim == 3 ? (int)(node / ((int64_t)n * n)) : 0 };
        for (int d = 0; d < dim; ++d) {
            float v = 0.0f;
            if (M != 0) {
                v = (float)((double)grid[(int64_t)(1 + d) * nodes + node] / (double)M);
                const float X = (float)idx[d] * dx;
                v = fminf(fmaxf(X + v, lo), hi) - X;
            }
            dg[(int64_t)d * nodes + node] = v;
            grid[(int64_t)(1 + d) * nodes + node] = 0;
        }
        grid[node] = 0;
    }
}

/*
 * particleIntegrate for an elastic material (section 3.3.2), without the
 * deformation update (oracle_update_F with dt = 1 does F <- (I + D) F): per
 * particle x_e <- x_e + d_e (float32), clamped to [dx, (n - 2) dx] with
 * clamped particles counted in status[2] (a backstop counted, not hidden);
 * then gravity goes into the next substep's displacement: d_e <- d_e + gdt2_e
 * with gdt2_e = g_e * (dt * dt) formed once in float32.
 */
void oracle_pbmpm_integrate(int dim, int n, int64_t np_, float *x, float *d, float dt, const float *gravity,
                            uint32_t *status)
{
    const float dx = 1.0f / (float)n;
    const float lo = dx, hi = (float)(n - 2) * dx;
    float gdt2[3];
    for (int e = 0; e < dim; ++e)
        gdt2[e] = gravity[e] * (dt * dt);
    for (int64_t p = 0; p < np_; ++p) {
        int clamped = 0;
        for (int e = 0; e < dim; ++e) {
            const float xa = x[(int64_t)e * np_ + p] + d[(int64_t)e * np_ + p];
            const float xc = fminf(fmaxf(xa, lo), hi);
            clamped |= xc != xa;
            x[(int64_t)e * np_ + p] = xc;
            d[(int64_t)e * np_ + p] = d[(int64_t)e * np_ + p] + gdt2[e];
        }
        status[ST_CLAMP] += (uint32_t)clamped;
    }
}
