"""Pins for the oracle's grid update, grid-to-particle gather and binning.

Grid update ("Implementation -- GPU Optimization & Reference Codebases",
section 1 four-phase step; section 2.1 consume-and-zero; section 5 rules 1,
4 and 7): integer accumulators are converted once, velocity is momentum over
mass, gravity is applied by the solver, and each accumulator is zeroed by its
one reader.  The sticky walls and the empty-node rule are the readings taken
for the dam-break substep (no page fixes them).

Gather (same page, sections 1 and 3.1; the APIC transfer): a particle reads
velocity and the affine matrix back from its stencil.  Closed form used: for
the quadratic B-spline the gather reproduces any affine velocity field
v(x) = A x + b exactly in real arithmetic, v_p = A x_p + b and
C_p = (4/dx^2) sum_i w_i v_i (x_i - x_p)^T = A, because
sum_i w_i (x_i - x_p)(x_i - x_p)^T = (dx^2/4) I.

Binning ("Particle worlds, part 3", steps 3 and 4; the implementation page's
section 2.1 on tiles): counting sort by cell = histogram, exclusive prefix sum,
scatter; cells are numbered tile by tile.
"""
from fractions import Fraction

import numpy as np
import pytest

from mpm_inputs import WORKLOADS, build, scaled
from mpm_inputs import generators as G

BIG = (1e30, 1e30, 1e30)


def particles(x, v, C, m):
    return {"x": np.ascontiguousarray(x, np.float32), "v": np.ascontiguousarray(v, np.float32),
            "C": np.ascontiguousarray(C, np.float32), "m": np.ascontiguousarray(m, np.float32)}


# ---------------------------------------------------------------- grid update

@pytest.mark.parametrize("dim", [2, 3])
def test_grid_update_velocity_gravity_walls_and_clear(oracle_lib, dim):
    n, sticky, dt = 8, 2, np.float32(1e-4)
    grav = np.array([0.0, -9.8, 0.0][:dim], np.float32)
    shape = (1 + dim,) + (n,) * dim
    grid = np.zeros(shape, np.int64)
    M = G.uniform_int(5, 1, n ** dim, 0, 1 << 40).reshape((n,) * dim)
    M.reshape(-1)[::7] = 0                                   # some empty nodes
    grid[0] = M
    for d in range(dim):
        grid[1 + d] = G.uniform_int(5, 2 + d, n ** dim, -(1 << 42), 1 << 42).reshape((n,) * dim)
    before = grid.copy()
    vg = oracle_lib.grid_update(dim, n, grid, float(dt), grav, sticky)
    assert np.all(grid == 0)                                  # consumed and zeroed
    gdt = [Fraction(float(np.float32(dt * grav[d]))) for d in range(dim)]
    for idx in np.ndindex(*(n,) * dim):
        wall = any(i < sticky or i >= n - sticky for i in idx)
        m = int(before[(0,) + idx])
        for d in range(dim):
            got = vg[(d,) + idx]
            if wall or m == 0:
                assert got == 0.0
                continue
            exact = Fraction(int(before[(1 + d,) + idx]), m) + gdt[d]
            # two float32 roundings (P/M, then the add) and one double rounding
            assert abs(Fraction(float(got)) - exact) <= abs(exact) * Fraction(3, 1 << 24) + Fraction(1, 1 << 40)


# ------------------------------------------------------------------- gather

@pytest.mark.parametrize("dim", [2, 3])
def test_gather_reproduces_affine_field(oracle_lib, dim):
    """Nodes carry v(x) = A x + b with a non-symmetric A: every interior
    particle gathers v = A x_p + b and C = A (not A^T, not a scaled A)."""
    n = 32
    dx = 1.0 / n
    A = np.array([[0.5, 3.0, -1.0], [-2.0, 0.25, 4.0], [1.5, -0.75, -0.5]])[:dim, :dim]
    b = np.array([0.1, -0.2, 0.3])[:dim]
    ax = np.arange(n) * dx
    mesh = np.meshgrid(*([ax] * dim), indexing="ij")
    tr = tuple(reversed(range(dim)))
    vg = np.stack([(sum(A[d, e] * mesh[e] for e in range(dim)) + b[d]).transpose(tr) for d in range(dim)])
    vg = np.ascontiguousarray(vg.astype(np.float32))
    N = 200
    x = 2.0 * dx + G.uniform01(7, 1, dim * N).reshape(dim, N) * (1.0 - 5.0 * dx)
    p = particles(x, np.zeros((dim, N)), np.zeros((dim * dim, N)), np.ones(N))
    x0 = p["x"].astype(np.float64).copy()
    dt = 1e-3
    status = oracle_lib.g2p(dim, n, vg, p, dt)
    assert status.tolist() == [0, 0, 0, 0]
    v_exact = A @ x0 + b[:, None]
    assert np.all(np.abs(p["v"] - v_exact) <= 2e-6 * (1 + np.abs(v_exact)))
    Cg = p["C"].astype(np.float64).reshape(dim, dim, N)
    assert np.all(np.abs(Cg - A[:, :, None]) <= 2e-3)          # fp32 B sums scaled by 4/dx^2
    # advection uses the new velocity: x = x0 + dt v
    assert np.all(np.abs(p["x"] - (x0 + dt * p["v"].astype(np.float64))) <= 2e-7)


def test_gather_clamps_and_counts(oracle_lib):
    n, dim = 16, 2
    dx = 1.0 / n
    vg = np.zeros((2, n, n), np.float32)
    vg[0] = -50.0                                               # strong flow toward x = 0
    x = np.array([[2.2 * dx, 8.0 * dx], [6.0 * dx, 6.0 * dx]])
    p = particles(x, np.zeros((2, 2)), np.zeros((4, 2)), np.ones(2))
    status = oracle_lib.g2p(dim, n, vg, p, 1e-2)
    assert status.tolist() == [0, 0, 2, 0]
    assert np.all(p["x"][0] == np.float32(dx))                  # clamped to the first interior node


@pytest.mark.parametrize("dim", [2, 3])
def test_substep_free_fall(oracle_lib, dim):
    """A block of particles moving with uniform velocity v0 and C = 0, away
    from the walls: after P2G -> grid update -> gather every particle moves
    with v0 + g dt and has C = 0 (constant-field reproduction), and the
    grid's total mass equals the particles' total."""
    n, k, sticky, dt = 32, 32, 2, 1e-3
    dx = 1.0 / n
    grav = [0.0, -9.8, 0.0][:dim]
    N = 500
    x = 10 * dx + G.uniform01(9, 1, dim * N).reshape(dim, N) * (10 * dx)
    v0 = np.array([0.3, -0.1, 0.2])[:dim]
    p = particles(x, np.repeat(v0[:, None], N, 1), np.zeros((dim * dim, N)), np.ones(N))
    grid, status = oracle_lib.p2g_quadratic(dim, n, k, p, BIG)
    assert abs(grid[0].sum() / 2.0 ** k - N) <= N * 3 ** dim * 2.0 ** -(k + 1) + N * 2.0 ** -20
    vg = oracle_lib.grid_update(dim, n, grid, dt, grav, sticky)
    oracle_lib.g2p(dim, n, vg, p, dt)
    want = v0 + np.float32(np.float32(dt) * np.float32(np.array(grav, np.float32)))
    assert np.all(np.abs(p["v"] - want[:, None]) <= 1e-6)
    assert np.all(np.abs(p["C"]) <= 5e-3)


# ------------------------------------------------------------------- binning

@pytest.mark.parametrize("name,count", [("pile_2d", None), ("dam_3d_128", 1 << 15), ("blobs_3d_256", 1 << 15)])
def test_binning_is_a_stable_counting_sort_by_tile_major_cell(oracle_lib, name, count):
    w = WORKLOADS[name] if count is None else scaled(WORKLOADS[name], count)
    p = build(w)
    x = p["x"]
    if name == "pile_2d":                                        # one particle out of the domain
        x[0, 3] = 0.0
    cnt, start, order = oracle_lib.bin_particles(w.dim, w.n, w.tile, p, (w.max_mass, w.max_speed, w.max_affine))
    valid = np.ones(w.n_particles, bool)
    if name == "pile_2d":
        valid[3] = False
    assert np.array_equal(np.sort(order), np.nonzero(valid)[0])  # a permutation of the kept particles
    assert start[0] == 0 and np.array_equal(start[1:], np.cumsum(cnt.astype(np.int64)))
    nt, t = w.n // w.tile, w.tile
    per = t ** w.dim
    g = x.astype(np.float64) * w.n
    for c in np.nonzero(cnt)[0]:
        members = order[start[c]:start[c + 1]]
        assert np.all(np.diff(members) > 0)                     # stable
        tile_id, local = divmod(int(c), per)
        base = []
        for e in range(w.dim):
            base.append((tile_id % nt) * t + local % t)
            tile_id //= nt
            local //= t
        for e in range(w.dim):
            ge = g[e, members]
            assert np.all((base[e] <= ge - 0.5) & (ge - 0.5 < base[e] + 1))
