"""Pins for the oracle's fixed-point APIC P2G with the quadratic B-spline.

What the pages fix and these tests check, independently of the oracle's own
arithmetic:
  - the shape function is a tensor product of 1D B-splines, non-negative,
    with partition of unity, and a second-order stencil sits on nodes
    {j-1, j, j+1} or {j, j+1, j+2} by whether the fractional coordinate is
    below one half ("Mass Matrix Assembly on Tensor Cores for Implicit PIC",
    shape-function section);
  - the APIC transfer deposits mass m w and momentum m w (v + C (x_i - x_p))
    ("Implementation -- GPU Optimization & Reference Codebases", section 3.1,
    APIC with the 3x3 quadratic stencil and affine matrix C);
  - accumulation is in rounded fixed point, so the grid is independent of
    particle order (same page, section 2.1 and rule 1 of section 5; rounding
    rather than truncating, section 3.3.1).
Closed forms used: the quadratic B-spline's values at distances 0, 1/2, 1,
3/2; its discrete moments sum_i w_i = 1, sum_i w_i (x_i - x_p) = 0 and
sum_i w_i (x_i - x_p)^2 = dx^2/4 (exact for this spline at any position),
which give the grid's mass and momentum moments in closed form; and a
brute-force evaluation of the textbook kernel by node distance over every
node of a tiny grid.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from mpm_inputs import WORKLOADS, build, scaled
from mpm_inputs import generators as G


def quad_bspline(t):
    """Textbook quadratic B-spline of a signed distance t (in cells), fp64."""
    a = np.abs(t)
    return np.where(a < 0.5, 0.75 - a * a, np.where(a < 1.5, 0.5 * (1.5 - a) ** 2, 0.0))


def particles(x, v, C, m):
    return {"x": np.ascontiguousarray(x, np.float32), "v": np.ascontiguousarray(v, np.float32),
            "C": np.ascontiguousarray(C, np.float32), "m": np.ascontiguousarray(m, np.float32)}


BIG = (1e30, 1e30, 1e30)  # declared ranges that reject nothing


def exact_node_values(dim, n, S, g, m, v, C, weights, base):
    """Exact rational node values for one particle whose 1D weights and
    offsets are given per axis."""
    dx = Fraction(1, n)
    out = {}
    idx = np.ndindex(*(3,) * dim)
    for o in idx:
        w = Fraction(m) * S
        for e in range(dim):
            w *= weights[o[e]]
        node = tuple(base[e] + o[e] for e in range(dim))
        r = [(base[e] + o[e]) * dx - Fraction(g[e]) * dx for e in range(dim)]
        vals = [w]
        for d in range(dim):
            u = Fraction(v[d]) + sum(Fraction(C[d][e]) * r[e] for e in range(dim))
            vals.append(w * u)
        out[node] = vals
    return out


@pytest.mark.parametrize("dim", [2, 3])
def test_particle_on_a_node(oracle_lib, dim):
    """At a node the 1D weights are N(1), N(0), N(1) = 1/8, 3/4, 1/8 on nodes
    j-1, j, j+1; with dyadic m, v, C every contribution is exact in float32,
    so the fixed-point grid equals the exact values bit for bit."""
    n, S = 64, 1 << 32
    g = [17, 9, 30][:dim]
    m = 1.25
    v = [0.5, -0.25, 2.0][:dim]
    C = [[0.125, -0.5, 1.0], [2.0, 0.375, -0.25], [-1.5, 0.75, 0.5]]
    C = [row[:dim] for row in C[:dim]]
    x = np.array([[gi / n] for gi in g])
    grid, status = oracle_lib.p2g_quadratic(dim, n, 32, particles(x, np.array([[vi] for vi in v]),
                                            np.array([[c] for row in C for c in row]), [m]), BIG)
    exp = exact_node_values(dim, n, S, g, m, v, C, [Fraction(1, 8), Fraction(3, 4), Fraction(1, 8)],
                            [gi - 1 for gi in g])
    expect = np.zeros_like(grid)
    for node, vals in exp.items():
        for ch, val in enumerate(vals):
            assert val.denominator == 1
            expect[(ch,) + tuple(reversed(node))] = int(val)
    assert np.array_equal(grid, expect)
    assert status.tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("dim", [2, 3])
def test_particle_half_way_between_nodes(oracle_lib, dim):
    """Fraction exactly 1/2: stencil {j, j+1, j+2} with weights 1/2, 1/2, 0."""
    n, S = 32, 1 << 20
    g = [Fraction(21, 2), Fraction(7, 2), Fraction(15, 2)][:dim]
    v = [1.0, -2.0, 0.5][:dim]
    C = [[0.0] * dim for _ in range(dim)]
    x = np.array([[float(gi) / n] for gi in g])
    grid, _ = oracle_lib.p2g_quadratic(dim, n, 20, particles(x, np.array([[vi] for vi in v]),
                                       np.zeros((dim * dim, 1)), [3.0]), BIG)
    exp = exact_node_values(dim, n, S, g, 3, v, C, [Fraction(1, 2), Fraction(1, 2), Fraction(0)],
                            [int(gi - Fraction(1, 2)) for gi in g])
    expect = np.zeros_like(grid)
    for node, vals in exp.items():
        for ch, val in enumerate(vals):
            expect[(ch,) + tuple(reversed(node))] = int(val)
    assert np.array_equal(grid, expect)


def brute_force_reference(dim, n, p):
    """Real-arithmetic (fp64) node mass and momentum by evaluating the
    textbook kernel on every node of the grid, plus per-node bounds on the
    magnitude of contributions and their count."""
    x, v, C, m = (p[k].astype(np.float64) for k in ("x", "v", "C", "m"))
    dx = 1.0 / n
    coords = np.meshgrid(*([np.arange(n) * dx] * dim), indexing="ij")  # coords[e][i_x, i_y, ...]
    M = np.zeros((n,) * dim)
    P = np.zeros((dim,) + (n,) * dim)
    A = np.zeros((n,) * dim)   # sum of |contribution| magnitudes (for the tolerance)
    K = np.zeros((n,) * dim)
    for q in range(m.shape[0]):
        w = np.ones((n,) * dim)
        for e in range(dim):
            w = w * quad_bspline((coords[e] - x[e, q]) / dx)
        M += m[q] * w
        mag = np.abs(np.ones_like(w))
        for d in range(dim):
            u = v[d, q] + sum(C[d * dim + e, q] * (coords[e] - x[e, q]) for e in range(dim))
            P[d] += m[q] * w * u
            mag = np.maximum(mag, np.abs(u))
        A += m[q] * w * mag
        K += w > 0
    # transpose from [i_x, i_y, i_z] to the grid's [z][y][x] layout
    tr = tuple(reversed(range(dim)))
    return M.transpose(tr), np.stack([P[d].transpose(tr) for d in range(dim)]), A.transpose(tr), K.transpose(tr)


@pytest.mark.parametrize("dim", [2, 3])
def test_brute_force_tiny_grid(oracle_lib, dim):
    """Node by node against the distance-evaluated kernel over the whole grid:
    |oracle/S - exact| <= 1e-5 * sum|contributions| + count * 2^-(k+1)."""
    n, k = 8, 32
    N = 12
    seed = 0xB0F
    x = 1.5 / n + G.uniform01(seed, 1, dim * N).reshape(dim, N) * ((n - 4.0) / n)
    v = G.normal(seed, 2, dim * N, 1.0).reshape(dim, N)
    C = G.normal(seed, 3, dim * dim * N, 3.0).reshape(dim * dim, N)
    m = 0.5 + G.uniform01(seed, 4, N)
    p = particles(x, v, C, m)
    grid, status = oracle_lib.p2g_quadratic(dim, n, k, p, BIG)
    assert status.tolist() == [0, 0, 0, 0]
    M, P, A, K = brute_force_reference(dim, n, p)
    S = 2.0 ** k
    tol = 1e-5 * A + K * 2.0 ** -(k + 1)
    assert np.all(np.abs(grid[0] / S - M) <= tol)
    for d in range(dim):
        assert np.all(np.abs(grid[1 + d] / S - P[d]) <= tol)
    assert np.all(grid[:, K == 0] == 0)      # nodes outside every stencil stay empty


def node_coords(dim, n):
    dx = 1.0 / n
    ax = np.arange(n) * dx
    mesh = np.meshgrid(*([ax] * dim), indexing="ij")
    tr = tuple(reversed(range(dim)))
    return [mesh[e].transpose(tr) for e in range(dim)]   # in the grid's [z][y][x] layout


def moment_checks(dim, n, k, grid, p):
    """Closed-form grid moments vs particle sums; returns (name, got, want, tol)."""
    S = 2.0 ** k
    dx = 1.0 / n
    x, v, C, m = (p[key].astype(np.float64) for key in ("x", "v", "C", "m"))
    cen = x.mean(axis=1)
    X = [c - cen[e] for e, c in enumerate(node_coords(dim, n))]
    xp = x - cen[:, None]
    Mg = grid[0].astype(np.float64) / S
    Pg = [grid[1 + d].astype(np.float64) / S for d in range(dim)]
    N = m.shape[0]
    umax = np.abs(v).max(axis=0) + np.abs(C).sum(axis=0) * 1.5 * dx
    ext = max(np.abs(xp).max() + 2 * dx, dx)
    # per-contribution error <= 1/2 quantum + 2^-19 relative, times |weight function|
    e_abs = N * 3 ** dim * 0.5 / S
    e_rel_m = 2.0 ** -19 * m.sum()
    e_rel_p = 2.0 ** -19 * (m * np.maximum(umax, 1.0)).sum()
    out = [("sum M", Mg.sum(), m.sum(), e_abs + e_rel_m)]
    for e in range(dim):
        out.append((f"sum M x{e}", (Mg * X[e]).sum(), (m * xp[e]).sum(), (e_abs + e_rel_m) * ext))
        for f in range(dim):
            want = (m * xp[e] * xp[f]).sum() + (m.sum() * dx * dx / 4 if e == f else 0.0)
            out.append((f"sum M x{e} x{f}", (Mg * X[e] * X[f]).sum(), want, (e_abs + e_rel_m) * ext * ext))
    for d in range(dim):
        out.append((f"sum P{d}", Pg[d].sum(), (m * v[d]).sum(), e_abs + e_rel_p))
        for e in range(dim):
            want = (m * (v[d] * xp[e] + C[d * dim + e] * dx * dx / 4)).sum()
            out.append((f"sum P{d} x{e}", (Pg[d] * X[e]).sum(), want, (e_abs + e_rel_p) * ext))
    return out


def _workload_cloud(name, n_particles=None):
    w = WORKLOADS[name]
    if n_particles is not None:
        w = scaled(w, n_particles)
    return w, build(w)


@pytest.mark.parametrize("name,count", [("pile_2d", None), ("dam_3d_128", 1 << 16), ("blobs_3d_256", 1 << 15)])
def test_grid_moments_on_workload_clouds(oracle_lib, name, count):
    w, p = _workload_cloud(name, count)
    grid, status = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, p, (w.max_mass, w.max_speed, w.max_affine))
    assert status.tolist() == [0, 0, 0, 0]
    for label, got, want, tol in moment_checks(w.dim, w.n, w.frac_bits, grid, p):
        assert abs(got - want) <= tol, (label, got, want, tol)


@pytest.mark.parametrize("dim", [2, 3])
def test_affine_term_enters_untransposed(oracle_lib, dim):
    """With v = 0 the momentum's first moment is sum_p m C dx^2/4 exactly in
    real arithmetic; a large non-symmetric C separates C from its transpose
    and from a dropped or sign-flipped affine term by far more than the
    rounding bound."""
    n, k, N = 32, 40, 64
    seed = 0xAFF
    x = 3.0 / n + G.uniform01(seed, 1, dim * N).reshape(dim, N) * ((n - 6.0) / n)
    C = G.normal(seed, 3, dim * dim * N, 50.0).reshape(dim * dim, N)
    C[1] += 200.0          # C_01 >> C_10 for every particle
    m = 1.0 + G.uniform01(seed, 4, N)
    p = particles(x, np.zeros((dim, N)), C, m)
    grid, _ = oracle_lib.p2g_quadratic(dim, n, k, p, BIG)
    checks = {lab: (got, want, tol) for lab, got, want, tol in moment_checks(dim, n, k, grid, p)}
    dx = 1.0 / n
    mm = p["m"].astype(np.float64)
    Cd = p["C"].astype(np.float64)
    for d in range(dim):
        for e in range(dim):
            got, want, tol = checks[f"sum P{d} x{e}"]
            assert abs(got - want) <= tol
            transposed = (mm * Cd[e * dim + d] * dx * dx / 4).sum()
            if d != e:
                assert abs(got - transposed) > 100 * tol


def test_partition_of_unity_per_particle(oracle_lib):
    """Each particle alone: the node masses sum to m*S within the rounding of
    its 27 contributions (1/2 quantum each) and float32 weight products."""
    n, k = 16, 30
    for i in range(60):
        x = 1.0 / n + G.uniform01(0xFACE, i, 3).reshape(3, 1) * ((n - 3.0) / n)
        grid, _ = oracle_lib.p2g_quadratic(3, n, k, particles(x, np.zeros((3, 1)), np.zeros((9, 1)), [1.0]), BIG)
        total = grid[0].sum()
        assert abs(total - 2 ** k) <= 27 * 0.5 + 2 ** k * 2.0 ** -20
        assert np.count_nonzero(grid[0]) <= 27 and np.all(grid[0] >= 0)


def test_grid_independent_of_particle_order(oracle_lib):
    w, p = _workload_cloud("dam_3d_128", 1 << 14)
    r = (w.max_mass, w.max_speed, w.max_affine)
    base, _ = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, p, r)
    N = w.n_particles
    for order in (G.permutation(1, 2, N), np.arange(N)[::-1].copy(), G.affine_order(N, 3, 7)):
        g, _ = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, p, r, order=order)
        assert np.array_equal(g, base)


def test_skipped_particles_are_counted(oracle_lib):
    w, p = _workload_cloud("pile_2d")
    r = (w.max_mass, w.max_speed, w.max_affine)
    q = {k: v.copy() for k, v in p.items()}
    q["x"][0, 5] = 0.0                 # base cell -1: outside the grid
    q["x"][1, 6] = np.nan
    q["x"][0, 7] = (w.n - 2.0) / w.n   # base n-3 is the last valid cell: kept
    q["v"][1, 8] = 100.0               # outside the declared speed range
    q["C"][3, 9] = -5.0                # outside the declared affine range
    q["m"][10] = np.inf
    grid, status = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, q, r)
    assert status.tolist() == [2, 3, 0, 0]
    keep = np.ones(w.n_particles, bool)
    keep[[5, 6, 8, 9, 10]] = False
    sub = {k: np.ascontiguousarray(v[..., keep]) for k, v in q.items()}
    g2, s2 = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, sub, r)
    assert s2.tolist() == [0, 0, 0, 0] and np.array_equal(grid, g2)


def test_bounds(oracle_lib):
    for name in ("pile_2d", "dam_3d_128", "blobs_3d_256", "dam_3d_256"):
        w = WORKLOADS[name]
        lb = oracle_lib.p2g_log2_bound(w.dim, w.n, w.frac_bits, w.n_particles, (w.max_mass, w.max_speed, w.max_affine))
        assert lb < 63, (name, lb)
    w = WORKLOADS["blobs_3d_256"]
    assert oracle_lib.p2g_log2_bound(3, 256, 40, 1 << 24, (2.0, 8.0, 0.5)) >= 63
    # closed form at a simple point: S=2^10, one particle, m=1, speed 1, no affine: (27/64) * 2^10 * (1+1e-6) + 1
    got = oracle_lib.p2g_log2_bound(3, 64, 10, 1, (1.0, 1.0, 0.0))
    assert math.isclose(got, math.log2(27 / 64 * 1024 * (1 + 1e-6) + 1), rel_tol=1e-12)


def test_quantiser_rounds_to_nearest_even(oracle_lib):
    """A particle on a node with m = 7/4 and S = 2^8 gives node values that
    are exact rationals with fractional parts 0, 1/4, 1/2 and 7/8 (e.g. the
    face node 7/4 * 256 * 9/128 = 31.5); the encode must round each to the
    nearest integer with ties to even (Python's round of a Fraction), not
    truncate.  Negative momentum checks the tie rule below zero."""
    n, k = 32, 8
    for v in (1.0, -1.0, 0.75):
        x = np.array([[9 / n], [11 / n], [13 / n]])
        grid, _ = oracle_lib.p2g_quadratic(3, n, k, particles(x, np.array([[v], [-v], [0.0]]), np.zeros((9, 1)),
                                                             [1.75]), BIG)
        exp = exact_node_values(3, n, 1 << k, [9, 11, 13], Fraction(7, 4), [Fraction(v), Fraction(-v), 0],
                                [[0] * 3] * 3, [Fraction(1, 8), Fraction(3, 4), Fraction(1, 8)], [8, 10, 12])
        fracs = set()
        for node, vals in exp.items():
            for ch, val in enumerate(vals):
                fracs.add(val - math.floor(val))
                assert grid[(ch,) + tuple(reversed(node))] == round(val), (node, ch, val)
        assert Fraction(1, 2) in fracs


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threaded_oracle_equals_single_thread(oracle_lib, threads):
    """The CPU baseline's all-cores leg (contiguous particle ranges, private
    grids, integer sums over the touched node tiles) gives the single-thread
    grid bit for bit, with skipped particles counted alike."""
    w = scaled(WORKLOADS["blobs_3d_256"], 1 << 15)
    host = build(w)
    host = {k: np.array(a, copy=True) for k, a in host.items()}
    host["x"][0, :7] = 1.5                     # outside the grid
    host["v"][1, 7:12] = 100.0                 # outside the declared ranges
    rng = (w.max_mass, w.max_speed, w.max_affine)
    ref, rst = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, host, rng)
    got, st = oracle_lib.p2g_quadratic_threads(w.dim, w.n, w.frac_bits, host, rng, threads)
    assert np.array_equal(got, ref)
    assert st.tolist() == rst.tolist() == [7, 5, 0, 0]
    order = np.arange(w.n_particles)[::-1].copy()
    got2, _ = oracle_lib.p2g_quadratic_threads(w.dim, w.n, w.frac_bits, host, rng, threads, order=order)
    assert np.array_equal(got2, ref)
