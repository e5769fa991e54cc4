"""Seeded synthetic particle clouds for the particle-to-grid (P2G) workloads.

This module holds only workload construction: random numbers, particle
placement and the per-workload constants.  It contains none of the transfer's
arithmetic (no weights, no stencils, no quantisation), so it can serve both the
CPU oracle and the HIP library without coupling them.

Random numbers come from SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based
generator: draw ``i`` of a stream is the SplitMix64 output function applied to
``base + (i + 1) * golden``.  Every derived distribution is written out here
(uniform from the top bits, normals by Box-Muller) instead of relying on a
library distribution whose algorithm could change between versions.  The
Box-Muller logarithm and cosine are evaluated here too (range reduction by
exact steps, then series in float64 with only IEEE-rounded +, -, *, /), not by
numpy's log and cos, whose vectorised versions differ in the last bit between
host CPUs: every host draws bit-identical inputs, so stored digests of results
on these inputs hold wherever the inputs are generated.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function, in place on a uint64 array."""
    t = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.right_shift(z, np.uint64(30), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M1, out=z)
        np.right_shift(z, np.uint64(27), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M2, out=z)
        np.right_shift(z, np.uint64(31), out=t); np.bitwise_xor(z, t, out=z)
    return z


_CHUNK = 1 << 20
_POOL = None


def _parallel(n: int, fn, out: np.ndarray) -> np.ndarray:
    """Fills out[lo:hi] = fn(lo, hi) over chunks on a small thread pool (numpy
    releases the GIL inside its loops).  Results do not depend on the pool."""
    global _POOL
    spans = [(lo, min(n, lo + _CHUNK)) for lo in range(0, n, _CHUNK)]
    if len(spans) <= 1:
        for lo, hi in spans:
            out[lo:hi] = fn(lo, hi)
        return out
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))

    def job(span):
        lo, hi = span
        out[lo:hi] = fn(lo, hi)
    list(_POOL.map(job, spans))
    return out


def _base(seed: int, tag: int) -> np.uint64:
    return _mix64(np.array([(seed * 0x100000001B3 + tag * 0x9E3779B1) & (2**64 - 1)], dtype=np.uint64))[0]


def _raw(base: np.uint64, lo: int, hi: int) -> np.ndarray:
    z = np.arange(lo + 1, hi + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        np.multiply(z, GOLDEN, out=z)
        np.add(z, base, out=z)
    return _mix64(z)


def stream_u64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """Draws ``start .. start+n-1`` of the stream named ``(seed, tag)``."""
    base = _base(seed, tag)
    return _parallel(n, lambda lo, hi: _raw(base, start + lo, start + hi), np.empty(n, dtype=np.uint64))


def _u01(base: np.uint64, lo: int, hi: int) -> np.ndarray:
    z = _raw(base, lo, hi)
    np.right_shift(z, np.uint64(11), out=z)
    return z.astype(np.float64) * 2.0**-53


def uniform01(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """float64 uniform on [0, 1) with 53 random bits."""
    base = _base(seed, tag)
    return _parallel(n, lambda lo, hi: _u01(base, start + lo, start + hi), np.empty(n, dtype=np.float64))


def uniform_int(seed: int, tag: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] (inclusive) by scaling 53 random bits."""
    span = hi - lo + 1
    return (lo + np.floor(uniform01(seed, tag, n) * span)).astype(np.int64)


_LN2 = 0.6931471805599453
_HALF_PI = 1.5707963267948966
_SQRT_HALF = 0.7071067811865476


def _log(y: np.ndarray) -> np.ndarray:
    """Natural logarithm of positive float64 y: y = m 2^e with m in
    [sqrt(1/2), sqrt(2)) (frexp and the doubling are exact), then
    ln m = 2 atanh(s) = 2 (s + s^3/3 + s^5/5 + ...), s = (m - 1)/(m + 1),
    |s| < 0.172, summed by Horner's rule to s^27 (truncation below 1e-20)."""
    m, e = np.frexp(y)
    low = m < _SQRT_HALF
    m = np.where(low, m * 2.0, m)
    e = e - low.astype(e.dtype)
    s = (m - 1.0) / (m + 1.0)
    z = s * s
    p = np.full_like(s, 1.0 / 27.0)
    for k in range(12, -1, -1):
        p = p * z + 1.0 / (2 * k + 1)
    return e.astype(np.float64) * _LN2 + 2.0 * s * p


def _cos_2pi(u: np.ndarray) -> np.ndarray:
    """cos(2 pi u) for float64 u in [0, 1): quadrant q = floor(4u) and
    f = 4u - q exactly (u holds 53-bit multiples of 2^-53), folded to
    f <= 1/2 by f -> 1 - f (cos and sin swap); then the Taylor series of cos
    and sin at phi = (pi/2) f <= pi/4, summed by Horner's rule to phi^26
    (truncation below 1e-20)."""
    v = u * 4.0
    q = np.floor(v)
    f = v - q
    fold = f > 0.5
    f = np.where(fold, 1.0 - f, f)
    phi = f * _HALF_PI
    z = phi * phi
    c = np.ones_like(phi)
    sn = np.ones_like(phi)
    for k in range(13, 0, -1):                 # cos: 1 - z/2! + z^2/4! ...; sin: phi (1 - z/3! + ...)
        c = 1.0 - z * c / ((2 * k - 1) * (2 * k))
        sn = 1.0 - z * sn / ((2 * k) * (2 * k + 1))
    sn = sn * phi
    cf = np.where(fold, sn, c)                 # cos((pi/2) f) before folding
    sf = np.where(fold, c, sn)                 # sin((pi/2) f)
    qi = q.astype(np.int64) & 3
    return np.where(qi == 0, cf, np.where(qi == 1, -sf, np.where(qi == 2, -cf, sf)))


def normal(seed: int, tag: int, n: int, sigma: float, start: int = 0) -> np.ndarray:
    """float64 normal draws N(0, sigma^2) by the Box-Muller transform: draw k
    uses uniforms k of streams (2*tag+1, 2*tag+2), r = sqrt(-2 ln(1-u1)),
    value = sigma * r * cos(2 pi u2) (ln and cos as _log and _cos_2pi)."""
    b1, b2 = _base(seed, 2 * tag + 1), _base(seed, 2 * tag + 2)

    def fn(lo, hi):
        u1 = _u01(b1, start + lo, start + hi)
        np.subtract(1.0, u1, out=u1)          # (0, 1]
        r = np.sqrt(_log(u1) * -2.0)
        c = _cos_2pi(_u01(b2, start + lo, start + hi))
        return (r * c) * sigma
    return _parallel(n, fn, np.empty(n, dtype=np.float64))


def permutation(seed: int, tag: int, n: int) -> np.ndarray:
    """A seeded shuffle of 0..n-1 (argsort of random 64-bit keys)."""
    return np.argsort(stream_u64(seed, tag, n), kind="stable").astype(np.int64)


def affine_order(n: int, a: int, b: int) -> np.ndarray:
    """The scrambled order (a*k + b) mod n, a permutation when gcd(a, n) == 1."""
    return ((np.arange(n, dtype=np.int64) * a + b) % n).astype(np.int64)


# ---------------------------------------------------------------------------
# Workload 1: integer cloud for the split cloud-in-cell scatter.
# ---------------------------------------------------------------------------

def integer_cloud(seed: int, n: int = 256, cells: int = 8, frac_bits: int = 16,
                  max_mass: int = 1000, max_speed: int = 1000) -> dict:
    """Positions in units of 2**-frac_bits cell uniform over a cells x cells
    grid, integer masses 1..max_mass and integer velocity components in
    [-max_speed, max_speed]."""
    span = cells << frac_bits
    X = np.stack([uniform_int(seed, 1, n, 0, span - 1), uniform_int(seed, 2, n, 0, span - 1)])
    m = uniform_int(seed, 3, n, 1, max_mass)
    vel = np.stack([uniform_int(seed, 4, n, -max_speed, max_speed),
                    uniform_int(seed, 5, n, -max_speed, max_speed)])
    return {
        "X": np.ascontiguousarray(X.astype(np.int32)),
        "m": np.ascontiguousarray(m.astype(np.int32)),
        "vel": np.ascontiguousarray(vel.astype(np.int32)),
        "cells": cells,
    }


def integer_cloud_quadratic(seed: int, n_particles: int, n: int, dim: int, max_mass: int, max_speed: int,
                            max_affine: int) -> dict:
    """Integer particles for the integer-split quadratic transfer: positions in
    units of 2^-16 cell uniform over [2, n-2) cells per axis, masses 1..max_mass,
    velocity components in [-max_speed, max_speed] and affine entries (velocity
    per cell) in [-max_affine, max_affine]."""
    X = np.stack([uniform_int(seed, 70 + e, n_particles, 2 << 16, ((n - 2) << 16) - 1) for e in range(dim)])
    m = uniform_int(seed, 75, n_particles, 1, max_mass)
    v = np.stack([uniform_int(seed, 76 + e, n_particles, -max_speed, max_speed) for e in range(dim)])
    C = np.stack([uniform_int(seed, 80 + q, n_particles, -max_affine, max_affine) for q in range(dim * dim)])
    return {"X": np.ascontiguousarray(X.astype(np.int32)), "m": np.ascontiguousarray(m.astype(np.int64)),
            "v": np.ascontiguousarray(v.astype(np.int64)), "C": np.ascontiguousarray(C.astype(np.int64))}


# ---------------------------------------------------------------------------
# Particle placements for the quadratic-stencil workloads.  Positions are in
# the unit domain with n nodes per axis, node i at i/n; "g" below is a
# coordinate in node units (g = x * n).
# ---------------------------------------------------------------------------

def _jittered_sites(seed: int, order_axes, n_sites: int, lo_cell: int, hi_cells, dim: int) -> np.ndarray:
    """Sites of a 2-per-cell-per-axis sub-lattice (spacing half a cell) filled
    in the given axis order (first axis slowest), each jittered uniformly by up
    to a quarter of the sub-lattice spacing.  Returns g coordinates [dim][n]."""
    counts = [None if hi is None else 2 * (hi - lo_cell) for hi in hi_cells]  # sub-sites per bounded axis
    k = np.arange(n_sites, dtype=np.int64)
    idx = [None] * dim
    # order_axes lists axes slowest -> fastest; the slowest axis is unbounded.
    rem = k
    for ax in reversed(order_axes[1:]):
        c = counts[ax]
        idx[ax] = rem % c
        rem = rem // c
    idx[order_axes[0]] = rem
    g = np.empty((dim, n_sites), dtype=np.float64)
    for ax in range(dim):
        jit = (uniform01(seed, 20 + ax, n_sites) - 0.5) * 0.25  # +-1/8 cell
        g[ax] = lo_cell + (idx[ax] + 0.5) * 0.5 + jit
    return g


def settled_pile_2d(seed: int, n_particles: int = 3500, n: int = 64) -> np.ndarray:
    """A flat-topped settled layer at the bottom of a 2D box: 4 particles per
    cell on a jittered sub-lattice over x-cells [2, n-2), filled row by row
    from y = 2 cells upward.  Returns x [2][N] in the unit domain."""
    g = _jittered_sites(seed, order_axes=[1, 0], n_sites=n_particles, lo_cell=2,
                        hi_cells=[n - 2, None], dim=2)
    return g / n


def dam_break_3d(seed: int, n_particles: int, n: int) -> np.ndarray:
    """A dam-break block in x < 0.5, y < 0.5: 8 particles per cell on a
    jittered 2x2x2 sub-lattice over cells [2, n/2) in x and y, filled in
    z-slowest order from z = 2 cells until n_particles sites are placed."""
    half = n // 2
    g = _jittered_sites(seed, order_axes=[2, 1, 0], n_sites=n_particles, lo_cell=2,
                        hi_cells=[half, half, None], dim=3)
    return g / n


def jelly_block_3d(seed: int, n_particles: int, n: int) -> np.ndarray:
    """An elastic cube resting just above the floor: 8 particles per cell on a
    jittered 2x2x2 sub-lattice, the cube side s cells with 8 s^3 = n_particles
    (n_particles must be 8 times a cube), centred in x and z, its bottom at
    y = 3 cells.  Returns x [3][N] in the unit domain."""
    s = round((n_particles / 8) ** (1.0 / 3.0))
    assert 8 * s ** 3 == n_particles and s + 6 <= n
    lo = [(n - s) // 2, 3, (n - s) // 2]
    k = np.arange(n_particles, dtype=np.int64)
    sub = [k % (2 * s), (k // (2 * s)) % (2 * s), k // (4 * s * s)]        # x fastest, then y, then z
    g = np.empty((3, n_particles), dtype=np.float64)
    for ax in range(3):
        jit = (uniform01(seed, 60 + ax, n_particles) - 0.5) * 0.25      # +-1/8 cell
        g[ax] = lo[ax] + (sub[ax] + 0.5) * 0.5 + jit
    return g / n


def gaussian_blobs_3d(seed: int, n_particles: int, n: int, n_blobs: int = 32,
                      sigma_cells: float = 4.0) -> np.ndarray:
    """n_blobs isotropic Gaussian blobs (sigma in cells) with seeded centres
    uniform in [n/8, 7n/8) per axis, n_particles/n_blobs samples each.
    Samples whose float32 node coordinate leaves [2, n-2) on any axis are
    redrawn from fresh counters."""
    per = n_particles // n_blobs
    assert per * n_blobs == n_particles
    centres = n / 8 + uniform01(seed, 40, 3 * n_blobs).reshape(n_blobs, 3) * (0.75 * n)
    blob = np.repeat(np.arange(n_blobs), per)
    g = np.empty((3, n_particles), dtype=np.float64)
    todo = np.arange(n_particles)
    ctr = 0
    while todo.size:
        draws = np.stack([normal(seed, 50 + ax, todo.size, sigma_cells, start=ctr) for ax in range(3)])
        ctr += todo.size
        cand = centres[blob[todo]].T + draws
        x32 = (cand / n).astype(np.float32)
        g32 = x32.astype(np.float64) * n
        ok = np.all((g32 >= 2.0) & (g32 < n - 2.0), axis=0)
        g[:, todo[ok]] = cand[:, ok]
        todo = todo[~ok]
    return g / n


def particle_fields(seed: int, n_particles: int, dim: int, mass, v_sigma: float, c_sigma: float) -> dict:
    """Velocity N(0, v_sigma^2) per component, affine matrix entries
    N(0, c_sigma^2), and mass (a constant, or a (lo, hi) uniform range)."""
    v = np.empty((dim, n_particles), dtype=np.float32)
    for d in range(dim):
        v[d] = normal(seed, 60 + d, n_particles, v_sigma)
    C = np.empty((dim * dim, n_particles), dtype=np.float32)
    for k in range(dim * dim):
        C[k] = normal(seed, 70 + k, n_particles, c_sigma)
    if isinstance(mass, tuple):
        lo, hi = mass
        m = (lo + (hi - lo) * uniform01(seed, 80, n_particles)).astype(np.float32)
    else:
        m = np.full(n_particles, float(mass), dtype=np.float32)
    return {"v": v, "C": C, "m": m}
