"""Pins for the oracle's integer-split cloud-in-cell scatter.

Source: "particle to grid transfer in checked integer arithmetic"
(integerc.dev), sections "integers do not care about order", "the program"
and "what the output shows": shares are made integers by splitting (far share
rounded once, near share the remainder), along x and then each part along y;
node totals equal particle totals as an identity; the grid is identical in
every particle order ((k*a + 13) mod 256 for odd a, reversed); a bounds line
stops the program before any scatter when the node bound does not fit I64.
"""
from fractions import Fraction

import numpy as np
import pytest

from mpm_inputs import WORKLOADS, build
from mpm_inputs import generators as G

W = WORKLOADS["cic_split_2d"]


@pytest.fixture(scope="module")
def cloud():
    return build(W)


def test_split_rounding_matches_exact_nearest_even(oracle_lib):
    """2,000+ random (q, f) plus every tie case: the far share is q*f/65536
    rounded to the nearest integer with ties to even (Python's round of an
    exact Fraction), the near share is the remainder."""
    q = G.uniform_int(11, 1, 2000, -(10**9), 10**9)
    f = G.uniform_int(11, 2, 2000, 0, 65535)
    cases = list(zip(q.tolist(), f.tolist()))
    # ties: q*f = 32768 (mod 65536) happens for f = 32768 and odd q, and f = 16384 with q = 2 mod 4, ...
    for qq in range(-41, 42):
        cases += [(qq, 32768), (qq, 16384), (qq, 49152), (qq, 8192)]
    for qq, ff in cases:
        far = oracle_lib.split_far(qq, ff)
        exact = Fraction(qq * ff, 65536)
        assert far == round(exact), (qq, ff)            # round() of a Fraction is half-to-even
        assert abs(far - exact) <= Fraction(1, 2)
        near = qq - far
        assert near + far == qq


def test_worked_example_with_ties(oracle_lib):
    """One particle of mass 3 at fraction (1/2, 1/4) of cell (3, 5), velocity
    (2, -1), worked by hand: mass 3 splits along x as far = round(1.5) = 2
    (tie to even), near = 1; the far part 2 splits along y as round(0.5) = 0
    (tie to even) -> (2, 0); the near part 1 as round(0.25) = 0 -> (1, 0).
    Momentum x = 6 splits as 3/3, then round(0.75) = 1 -> (2, 1) for both
    parts; momentum y = -3 splits as far = round(-1.5) = -2, near = -1, then
    round(-0.5) = 0 -> (-2, 0) and round(-0.25) = 0 -> (-1, 0)."""
    X = np.array([[3 * 65536 + 32768], [5 * 65536 + 16384]], dtype=np.int32)
    m = np.array([3], dtype=np.int32)
    vel = np.array([[2], [-1]], dtype=np.int32)
    grid, status = oracle_lib.p2g_cic_split(X, m, vel, 8)
    expect = np.zeros((3, 9, 9), dtype=np.int64)
    # [channel][y][x]
    expect[0, 5, 3], expect[0, 6, 3], expect[0, 5, 4], expect[0, 6, 4] = 1, 0, 2, 0
    expect[1, 5, 3], expect[1, 6, 3], expect[1, 5, 4], expect[1, 6, 4] = 2, 1, 2, 1
    expect[2, 5, 3], expect[2, 6, 3], expect[2, 5, 4], expect[2, 6, 4] = -1, 0, -2, 0
    assert np.array_equal(grid, expect)
    assert status.tolist() == [0, 0, 0, 0]


def test_totals_are_an_identity(oracle_lib, cloud):
    grid, status = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n)
    m = cloud["m"].astype(np.int64)
    assert grid[0].sum() == m.sum()
    assert grid[1].sum() == (m * cloud["vel"][0]).sum()
    assert grid[2].sum() == (m * cloud["vel"][1]).sum()
    assert status[0] == 0


def test_every_scrambled_order_gives_the_same_grid(oracle_lib, cloud):
    base, _ = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n)
    n = W.n_particles
    orders = [G.affine_order(n, a, 13) for a in range(1, 256, 2)]
    orders += [np.arange(n)[::-1].copy(), G.affine_order(n, 97, 200)]
    orders += [G.permutation(W.seed ^ 0x5F5F, 100 + s, n) for s in range(3)]
    for o in orders:
        g, _ = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n, order=o)
        assert np.array_equal(g, base)


def test_nodes_within_one_unit_per_particle_of_exact_bilinear(oracle_lib, cloud):
    """Each particle's share at a node differs from the exact bilinear share
    q * wx * wy by at most 1 (1/2 from the x split carried through a weight
    <= 1, plus 1/2 from the y split), so a node is within its contributor
    count of the exact rational sum."""
    grid, _ = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n)
    X, m, vel = cloud["X"].astype(np.int64), cloud["m"].astype(np.int64), cloud["vel"].astype(np.int64)
    exact = np.zeros((3, 9, 9), dtype=object)
    count = np.zeros((9, 9), dtype=np.int64)
    for p in range(W.n_particles):
        cx, fx = divmod(int(X[0, p]), 65536)
        cy, fy = divmod(int(X[1, p]), 65536)
        q = [int(m[p]), int(m[p] * vel[0, p]), int(m[p] * vel[1, p])]
        for i, wx in ((0, 65536 - fx), (1, fx)):
            for j, wy in ((0, 65536 - fy), (1, fy)):
                count[cy + j, cx + i] += 1
                for c in range(3):
                    exact[c, cy + j, cx + i] += Fraction(q[c] * wx * wy, 1 << 32)
    for c in range(3):
        for yy in range(9):
            for xx in range(9):
                assert abs(grid[c, yy, xx] - exact[c, yy, xx]) <= count[yy, xx]


def test_bounds_line(oracle_lib):
    assert oracle_lib.cic_bounds_ok(256, 1000, 1000)
    assert not oracle_lib.cic_bounds_ok(1 << 40, 1 << 20, 1 << 20)
    assert not oracle_lib.cic_bounds_ok(1, 1 << 40, 1 << 20)   # q * f would overflow


def test_out_of_domain_particles_are_skipped_and_counted(oracle_lib, cloud):
    X = cloud["X"].copy()
    X[0, 7] = 8 * 65536          # one past the last cell
    X[1, 9] = -1
    g, status = oracle_lib.p2g_cic_split(X, cloud["m"], cloud["vel"], W.n)
    keep = np.ones(W.n_particles, bool)
    keep[[7, 9]] = False
    g2, s2 = oracle_lib.p2g_cic_split(np.ascontiguousarray(cloud["X"][:, keep]), cloud["m"][keep],
                                      np.ascontiguousarray(cloud["vel"][:, keep]), W.n)
    assert status[0] == 2 and s2[0] == 0
    assert np.array_equal(g, g2)


def test_float_scatter_is_order_dependent_integer_is_not(oracle_lib, cloud):
    """The page's contrast, on this cloud: the same bilinear scatter summed in
    float32 changes with the particle order, the integer split does not."""
    X, m, vel = cloud["X"].astype(np.int64), cloud["m"].astype(np.float32), cloud["vel"].astype(np.float32)

    def float_grid(order):
        g = np.zeros((9, 9), dtype=np.float32)
        for p in order:
            cx, fx = divmod(int(X[0, p]), 65536)
            cy, fy = divmod(int(X[1, p]), 65536)
            wx1, wy1 = np.float32(fx / 65536), np.float32(fy / 65536)
            q = m[p] * vel[0, p]
            for i, wx in ((0, np.float32(1) - wx1), (1, wx1)):
                for j, wy in ((0, np.float32(1) - wy1), (1, wy1)):
                    g[cy + j, cx + i] = np.float32(g[cy + j, cx + i] + np.float32(q * wx) * wy)
        return g
    a = float_grid(range(W.n_particles))
    b = float_grid(G.affine_order(W.n_particles, 97, 13))
    assert np.count_nonzero(a != b) > 0
    gi, _ = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n)
    gj, _ = oracle_lib.p2g_cic_split(cloud["X"], cloud["m"], cloud["vel"], W.n,
                                     order=G.affine_order(W.n_particles, 97, 13))
    assert np.array_equal(gi, gj)
