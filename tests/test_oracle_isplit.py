"""Pins for the oracle's integer-split quadratic APIC transfer.

"particle to grid transfer in checked integer arithmetic", sections "integers
do not care about order" and "what is not claimed": a quantity is split
between nodes with the far shares rounded once and the near share taking the
rest, so node totals equal particle totals exactly in every order; quadratic
weights and the affine term "would be more splits of the same kind".  The
quadratic B-spline weights and the first moments w_o (o - f) are exact dyadic
rationals at positions given in 2^-16 cell.

Pins, none of which re-types the oracle's arithmetic: exact conservation of
mass and momentum (an identity), identical grids in every particle order,
every node within the rounding bound of the exact rational APIC transfer
(Fraction arithmetic on tiny clouds), a particle on a node in closed form,
the tie rule, the bounds line and counted out-of-domain particles.
"""
from fractions import Fraction

import numpy as np
import pytest

from mpm_inputs import WORKLOADS, build
from mpm_inputs import generators as G


def cloud(dim, n, np_, seed, mm=1000, vv=1000, cc=1000):
    return G.integer_cloud_quadratic(seed, np_, n, dim, mm, vv, cc)


@pytest.mark.parametrize("name", ["isplit_2d_64", "isplit_3d_128"])
def test_node_totals_equal_particle_totals_exactly(oracle_lib, name):
    w = WORKLOADS[name]
    h = build(w) if w.dim == 2 else cloud(3, w.n, 20000, w.seed)
    g, st = oracle_lib.p2g_isplit(w.dim, w.n, h)
    assert st.tolist() == [0, 0, 0, 0]
    assert int(g[0].sum()) == int(h["m"].sum())
    for d in range(w.dim):
        assert int(g[1 + d].sum()) == int((h["m"] * h["v"][d]).sum())


@pytest.mark.parametrize("dim", [2, 3])
def test_identical_in_every_order(oracle_lib, dim):
    n = 16 if dim == 3 else 32
    h = cloud(dim, n, 3000, 0x15 + dim)
    base, _ = oracle_lib.p2g_isplit(dim, n, h)
    N = h["m"].shape[0]
    for order in [np.arange(N)[::-1].copy(), G.permutation(7, 1, N), G.affine_order(N, 773, 13)]:
        g, _ = oracle_lib.p2g_isplit(dim, n, h, order=order)
        assert np.array_equal(g, base)


def exact_transfer(dim, n, h):
    """The real-valued APIC transfer in exact rationals: m w_i (v + C (i - g)),
    with the textbook quadratic B-spline evaluated by distance."""
    def N(t):
        t = abs(t)
        if t < Fraction(1, 2):
            return Fraction(3, 4) - t * t
        if t < Fraction(3, 2):
            return (Fraction(3, 2) - t) ** 2 / 2
        return Fraction(0)
    np_ = h["m"].shape[0]
    out = {}
    for p in range(np_):
        g = [Fraction(int(h["X"][e][p]), 65536) for e in range(dim)]
        base = [int((g[e] - Fraction(1, 2)) // 1) for e in range(dim)]
        m = int(h["m"][p])
        rng = [range(base[e], base[e] + 3) for e in range(dim)]
        idxs = [(i, j) for i in rng[0] for j in rng[1]] if dim == 2 else \
               [(i, j, k) for i in rng[0] for j in rng[1] for k in rng[2]]
        for node in idxs:
            wgt = Fraction(1)
            for e in range(dim):
                wgt *= N(node[e] - g[e])
            vals = [m * wgt]
            for d in range(dim):
                u = Fraction(int(h["v"][d][p]))
                for e in range(dim):
                    u += int(h["C"][d * dim + e][p]) * (node[e] - g[e])
                vals.append(m * wgt * u)
            acc = out.setdefault(node, [Fraction(0)] * (1 + dim) + [0])
            for c in range(1 + dim):
                acc[c] += vals[c]
            acc[-1] += 1
    return out


@pytest.mark.parametrize("dim", [2, 3])
def test_within_rounding_of_exact_transfer(oracle_lib, dim):
    """Each tensor split of a quantity moves each of its node shares by at most
    dim from the exact value (a rounded outer share errs by 1/2, the middle by
    1, and later splits scale earlier errors by weights below 1); momentum is
    1 + dim splits.  So |integer - exact| <= contributors * (1 + dim) * dim."""
    n = 8
    h = cloud(dim, n, 60 if dim == 3 else 150, 0x77 + dim, mm=50, vv=40, cc=30)
    g, st = oracle_lib.p2g_isplit(dim, n, h)
    assert st.tolist() == [0, 0, 0, 0]
    ex = exact_transfer(dim, n, h)
    assert len(ex) > 0
    for node, acc in ex.items():
        idx = tuple(reversed(node))                      # grid is [c][z][y][x] / [c][y][x]
        cnt = acc[-1]
        assert abs(g[(0,) + idx] - acc[0]) <= cnt * dim
        for d in range(dim):
            assert abs(g[(1 + d,) + idx] - acc[1 + d]) <= cnt * (1 + dim) * dim
    touched = {tuple(reversed(i)) for i in ex}
    nz = {tuple(int(t) for t in i) for i in np.argwhere((g != 0).any(axis=0))}
    assert nz <= touched


def test_particle_on_a_node_closed_form(oracle_lib):
    """g = node + 1 (f = 1): weights (1/8, 3/4, 1/8), first moments
    (-1/8, 0, 1/8); quantities divisible by 64 split exactly (2D)."""
    dim, n = 2, 8
    h = {"X": np.array([[3 << 16], [4 << 16]], np.int32), "m": np.array([64], np.int64),
         "v": np.array([[2], [-1]], np.int64), "C": np.array([[8], [0], [0], [-4]], np.int64)}
    g, st = oracle_lib.p2g_isplit(dim, n, h)
    w = [Fraction(1, 8), Fraction(3, 4), Fraction(1, 8)]
    u = [Fraction(-1, 8), Fraction(0), Fraction(1, 8)]
    for a in range(3):
        for b in range(3):
            node = (3 + b, 2 + a)                         # [y][x]: base x = 2, base y = 3
            assert g[(0,) + node] == 64 * w[a] * w[b]
            assert g[(1,) + node] == 64 * 2 * w[a] * w[b] + 64 * 8 * u[a] * w[b]
            assert g[(2,) + node] == 64 * -1 * w[a] * w[b] + 64 * -4 * w[a] * u[b]


def test_ties_round_to_even(oracle_lib):
    """f = 1/2 (F = 2^15): w = (1/2, 1/2, 0); q w0 = q/2 is a tie for odd q."""
    dim, n = 2, 8
    for q, far in [(1, 0), (3, 2), (5, 2), (7, 4)]:
        h = {"X": np.array([[(2 << 16) + (1 << 15)], [4 << 16]], np.int32), "m": np.array([q], np.int64),
             "v": np.zeros((2, 1), np.int64), "C": np.zeros((4, 1), np.int64)}
        g, _ = oracle_lib.p2g_isplit(dim, n, h)
        # x: base 2, F = 2^15 -> shares (q/2 rounded even, rest, 0); y: f = 1 -> (1/8, 3/4, 1/8) of each
        col0 = g[0][:, 2].sum()
        col1 = g[0][:, 3].sum()
        assert (col0, col1, g[0][:, 4].sum()) == (far, q - far, 0)


def test_bounds_and_domain(oracle_lib):
    assert oracle_lib.isplit_bounds_ok(3, 1 << 20, 1000, 1000, 1000)
    assert not oracle_lib.isplit_bounds_ok(3, 1 << 40, 1 << 20, 1 << 20, 1 << 20)
    # the affine term counts: 2^40 (1 + 1) fits; with 3 entries of 2^20 at the line's allowance of 3/2 each
    # (first-moment shares sum to at most 1/2 in magnitude, doubled by the middle taking the rest, plus
    # rounding) it does not
    assert oracle_lib.isplit_bounds_ok(3, 1 << 20, 1 << 20, 1, 0)
    assert not oracle_lib.isplit_bounds_ok(3, 1 << 20, 1 << 20, 1, 1 << 20)
    dim, n = 3, 8
    # particle 0: x = 1/2 - 2^-16 cell puts its base node at -1; particle 1: z = n - 1 puts it at n - 2
    h = {"X": np.array([[(1 << 15) - 1, 3 << 16], [3 << 16, 3 << 16], [3 << 16, (n - 1) << 16]], np.int32),
         "m": np.array([1, 1], np.int64), "v": np.zeros((3, 2), np.int64), "C": np.zeros((9, 2), np.int64)}
    g, st = oracle_lib.p2g_isplit(dim, n, h)
    assert st.tolist() == [2, 0, 0, 0] and int(np.abs(g).sum()) == 0
    # the last positions inside: base 0 at x = 1/2 and base n - 3 just below x = n - 3/2
    h["X"][0] = [1 << 15, (n << 16) - 3 * (1 << 15) - 1]
    h["X"][2] = [3 << 16, 3 << 16]
    h["m"][:] = 64
    g, st = oracle_lib.p2g_isplit(dim, n, h)
    assert st.tolist() == [0, 0, 0, 0] and int(g[0].sum()) == 128
    assert g[0][:, :, 0].sum() > 0 and g[0][:, :, n - 1].sum() > 0
