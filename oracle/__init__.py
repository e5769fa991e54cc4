"""CPU oracle for the P2G transfer and its neighbouring steps.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the library's product path.
It shares no code with the HIP library (see mpm_oracle.c for the definitions
and the pages each step follows).

``build()`` compiles mpm_oracle.c with gcc; the wrappers below take numpy
arrays and return numpy arrays.
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mpm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmpm_oracle.so")
_lib = None

I64P = ct.POINTER(ct.c_int64)
U32P = ct.POINTER(ct.c_uint32)
I32P = ct.POINTER(ct.c_int32)
F32P = ct.POINTER(ct.c_float)


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libmpm_oracle.so (plain gcc, -O2,
    no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
                        "-fopenmp", "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ct.CDLL(_LIB_PATH)
        L.oracle_split_far.restype = ct.c_int64
        L.oracle_split_far.argtypes = [ct.c_int64, ct.c_int32]
        L.oracle_cic_bounds_ok.restype = ct.c_int
        L.oracle_cic_bounds_ok.argtypes = [ct.c_int64, ct.c_int64, ct.c_int64]
        L.oracle_p2g_cic_split.restype = None
        L.oracle_p2g_cic_split.argtypes = [ct.c_int64, I32P, I32P, I32P, I64P, ct.c_int32, I64P, U32P]
        L.oracle_p2g_quadratic.restype = None
        L.oracle_p2g_quadratic.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_int64, F32P, F32P, F32P, F32P,
                                           I64P, ct.c_double, ct.c_double, ct.c_double, I64P, U32P]
        L.oracle_p2g_quadratic_threads.restype = ct.c_int
        L.oracle_p2g_quadratic_threads.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_int64, F32P, F32P, F32P, F32P,
                                                   I64P, ct.c_double, ct.c_double, ct.c_double, I64P, U32P,
                                                   ct.c_int]
        L.oracle_pbmpm_project_elastic.restype = None
        L.oracle_pbmpm_project_elastic.argtypes = [ct.c_int, ct.c_int64, F32P, F32P, ct.c_float, ct.c_int, U32P]
        L.oracle_pbmpm_grid_update.restype = None
        L.oracle_pbmpm_grid_update.argtypes = [ct.c_int, ct.c_int, I64P, F32P, ct.c_int]
        L.oracle_pbmpm_integrate.restype = None
        L.oracle_pbmpm_integrate.argtypes = [ct.c_int, ct.c_int, ct.c_int64, F32P, F32P, ct.c_float, F32P, U32P]
        L.oracle_p2g_log2_bound.restype = ct.c_double
        L.oracle_p2g_log2_bound.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_int64,
                                            ct.c_double, ct.c_double, ct.c_double]
        L.oracle_grid_update.restype = None
        L.oracle_grid_update.argtypes = [ct.c_int, ct.c_int, I64P, F32P, ct.c_float, F32P, ct.c_int]
        L.oracle_g2p.restype = None
        L.oracle_g2p.argtypes = [ct.c_int, ct.c_int, F32P, ct.c_int64, F32P, F32P, F32P, ct.c_float, U32P]
        L.oracle_bin.restype = ct.c_int64
        L.oracle_p2g_isplit.argtypes = [ct.c_int, ct.c_int, ct.c_int64, I32P, I64P, I64P, I64P, I64P, I64P, U32P]
        L.oracle_isplit_bounds_ok.restype = ct.c_int
        L.oracle_isplit_bounds_ok.argtypes = [ct.c_int, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64]
        L.oracle_neohookean_affine.argtypes = [ct.c_int, ct.c_int, ct.c_int64, F32P, F32P, F32P, F32P, ct.c_float,
                                               ct.c_float, ct.c_float, F32P, U32P]
        L.oracle_update_F.argtypes = [ct.c_int, ct.c_int64, F32P, F32P, ct.c_float]
        L.oracle_bin.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_int64, F32P, F32P, F32P, F32P,
                                 ct.c_double, ct.c_double, ct.c_double, U32P, U32P, I64P]
        _lib = L
    return _lib


def _p(a: np.ndarray, ctype):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctype)


def _order_ptr(order):
    if order is None:
        return None, None
    o = np.ascontiguousarray(order, dtype=np.int64)
    return o, _p(o, I64P)


def split_far(q: int, f: int) -> int:
    return lib().oracle_split_far(int(q), int(f))


def cic_bounds_ok(n: int, max_mass: int, max_speed: int) -> bool:
    return bool(lib().oracle_cic_bounds_ok(n, max_mass, max_speed))


def p2g_cic_split(X, m, vel, cells: int, order=None):
    """Integer-split cloud-in-cell scatter; returns (grid[3][cells+1][cells+1], status[4])."""
    X = np.ascontiguousarray(X, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.int32)
    vel = np.ascontiguousarray(vel, dtype=np.int32)
    n = m.shape[0]
    grid = np.zeros((3, cells + 1, cells + 1), dtype=np.int64)
    status = np.zeros(4, dtype=np.uint32)
    o, op = _order_ptr(order)
    lib().oracle_p2g_cic_split(n, _p(X, I32P), _p(m, I32P), _p(vel, I32P), op, cells, _p(grid, I64P),
                               _p(status, U32P))
    return grid, status


def _soa(d):
    return (np.ascontiguousarray(d["x"], dtype=np.float32), np.ascontiguousarray(d["v"], dtype=np.float32),
            np.ascontiguousarray(d["C"], dtype=np.float32), np.ascontiguousarray(d["m"], dtype=np.float32))


def p2g_quadratic(dim: int, n: int, frac_bits: int, particles: dict, ranges, order=None, grid=None):
    """Fixed-point APIC P2G; returns (grid[1+dim][n]*dim, status[4])."""
    x, v, C, m = _soa(particles)
    np_ = m.shape[0]
    shape = (1 + dim,) + (n,) * dim
    if grid is None:
        grid = np.zeros(shape, dtype=np.int64)
    status = np.zeros(4, dtype=np.uint32)
    o, op = _order_ptr(order)
    lib().oracle_p2g_quadratic(dim, n, frac_bits, np_, _p(x, F32P), _p(v, F32P), _p(C, F32P), _p(m, F32P), op,
                               float(ranges[0]), float(ranges[1]), float(ranges[2]), _p(grid, I64P),
                               _p(status, U32P))
    return grid, status


def p2g_quadratic_threads(dim: int, n: int, frac_bits: int, particles: dict, ranges, threads: int, order=None,
                          grid=None):
    """The same P2G on `threads` host threads (private grids, integer-summed);
    bit-identical to p2g_quadratic.  For the CPU baseline's all-cores leg."""
    x, v, C, m = _soa(particles)
    np_ = m.shape[0]
    shape = (1 + dim,) + (n,) * dim
    if grid is None:
        grid = np.zeros(shape, dtype=np.int64)
    status = np.zeros(4, dtype=np.uint32)
    o, op = _order_ptr(order)
    rc = lib().oracle_p2g_quadratic_threads(dim, n, frac_bits, np_, _p(x, F32P), _p(v, F32P), _p(C, F32P),
                                            _p(m, F32P), op, float(ranges[0]), float(ranges[1]), float(ranges[2]),
                                            _p(grid, I64P), _p(status, U32P), int(threads))
    if rc != 0:
        raise MemoryError("oracle_p2g_quadratic_threads: private grids could not be allocated")
    return grid, status


def p2g_log2_bound(dim, n, frac_bits, np_, ranges) -> float:
    return lib().oracle_p2g_log2_bound(dim, n, frac_bits, np_, float(ranges[0]), float(ranges[1]),
                                       float(ranges[2]))


def grid_update(dim: int, n: int, grid: np.ndarray, dt: float, gravity, sticky: int):
    """Consumes (and zeroes) grid in place; returns vg[dim][n]*dim."""
    assert grid.dtype == np.int64 and grid.flags.c_contiguous
    vg = np.zeros((dim,) + (n,) * dim, dtype=np.float32)
    g = np.zeros(3, dtype=np.float32)
    g[:dim] = np.asarray(gravity, dtype=np.float32)[:dim]
    lib().oracle_grid_update(dim, n, _p(grid, I64P), _p(vg, F32P), ct.c_float(dt), _p(g, F32P), sticky)
    return vg


def g2p(dim: int, n: int, vg: np.ndarray, particles: dict, dt: float):
    """Updates particles['x'], ['v'], ['C'] in place; returns status[4]."""
    x, v, C, _ = _soa(particles)
    assert x is particles["x"] and v is particles["v"] and C is particles["C"], "arrays must be float32 C-contiguous"
    vg = np.ascontiguousarray(vg, dtype=np.float32)
    status = np.zeros(4, dtype=np.uint32)
    lib().oracle_g2p(dim, n, _p(vg, F32P), x.shape[1], _p(x, F32P), _p(v, F32P), _p(C, F32P), ct.c_float(dt),
                     _p(status, U32P))
    return status


def p2g_isplit(dim: int, n: int, particles: dict, order=None, grid=None):
    """Integer-split quadratic APIC transfer; particles: X int32 [dim][np] (2^-16 cell), m int64 [np],
    v int64 [dim][np], C int64 [dim*dim][np].  Returns (grid int64 [1+dim][n]*dim, status[4])."""
    X = np.ascontiguousarray(particles["X"], dtype=np.int32)
    m = np.ascontiguousarray(particles["m"], dtype=np.int64)
    v = np.ascontiguousarray(particles["v"], dtype=np.int64)
    C = np.ascontiguousarray(particles["C"], dtype=np.int64)
    np_ = m.shape[0]
    if grid is None:
        grid = np.zeros((1 + dim,) + (n,) * dim, dtype=np.int64)
    status = np.zeros(4, dtype=np.uint32)
    o, op = _order_ptr(order)
    lib().oracle_p2g_isplit(dim, n, np_, _p(X, I32P), _p(m, I64P), _p(v, I64P), _p(C, I64P), op, _p(grid, I64P),
                            _p(status, U32P))
    return grid, status


def isplit_bounds_ok(dim: int, np_: int, max_mass: int, max_speed: int, max_affine: int) -> bool:
    return bool(lib().oracle_isplit_bounds_ok(dim, np_, max_mass, max_speed, max_affine))


def neohookean_affine(dim: int, n: int, particles: dict, F: np.ndarray, vol0: np.ndarray, dt: float, mu: float,
                      lam: float):
    """MLS-MPM affine matrix with the Neo-Hookean stress term; returns (C'[dim*dim][np], status[4])."""
    _, _, C, m = _soa(particles)
    F = np.ascontiguousarray(F, dtype=np.float32)
    vol0 = np.ascontiguousarray(vol0, dtype=np.float32)
    out = np.empty_like(C)
    status = np.zeros(4, dtype=np.uint32)
    lib().oracle_neohookean_affine(dim, n, m.shape[0], _p(F, F32P), _p(C, F32P), _p(m, F32P), _p(vol0, F32P),
                                   ct.c_float(dt), ct.c_float(mu), ct.c_float(lam), _p(out, F32P), _p(status, U32P))
    return out, status


def update_F(dim: int, C: np.ndarray, F: np.ndarray, dt: float) -> None:
    """F <- (I + dt C) F in place (F float32 C-contiguous [dim*dim][np])."""
    C = np.ascontiguousarray(C, dtype=np.float32)
    assert F.dtype == np.float32 and F.flags.c_contiguous
    lib().oracle_update_F(dim, F.shape[1], _p(C, F32P), _p(F, F32P), ct.c_float(dt))


def bin_particles(dim: int, n: int, tile: int, particles: dict, ranges):
    """Counting sort by tile-major cell key; returns (cell_count, cell_start, order)."""
    x, v, C, m = _soa(particles)
    np_ = m.shape[0]
    n_cells = n ** dim
    count = np.zeros(n_cells, dtype=np.uint32)
    start = np.zeros(n_cells + 1, dtype=np.uint32)
    order = np.zeros(max(np_, 1), dtype=np.int64)
    placed = lib().oracle_bin(dim, n, tile, np_, _p(x, F32P), _p(v, F32P), _p(C, F32P), _p(m, F32P),
                              float(ranges[0]), float(ranges[1]), float(ranges[2]), _p(count, U32P),
                              _p(start, U32P), _p(order, I64P))
    return count, start, order[:placed]


# ------------------------------------------------------------------ PB-MPM

def pbmpm_project_elastic(dim: int, F: np.ndarray, D: np.ndarray, relax: float, polar_iters: int):
    """Elastic projection of D (float32 [dim*dim][np], updated in place) toward
    the polar rotation of (I + D) F; returns status[4]."""
    F = np.ascontiguousarray(F, dtype=np.float32)
    assert D.dtype == np.float32 and D.flags.c_contiguous
    status = np.zeros(4, dtype=np.uint32)
    lib().oracle_pbmpm_project_elastic(dim, D.shape[-1], _p(F, F32P), _p(D, F32P), ct.c_float(relax), polar_iters,
                                       _p(status, U32P))
    return status


def pbmpm_grid_update(dim: int, n: int, grid: np.ndarray, band: int):
    """Displacement-form grid update; consumes (zeroes) grid; returns dg[dim][n]*dim."""
    assert grid.dtype == np.int64 and grid.flags.c_contiguous
    dg = np.zeros((dim,) + (n,) * dim, dtype=np.float32)
    lib().oracle_pbmpm_grid_update(dim, n, _p(grid, I64P), _p(dg, F32P), band)
    return dg


def pbmpm_integrate(dim: int, n: int, x: np.ndarray, d: np.ndarray, dt: float, gravity):
    """x += d (clamped, counted in status[2]), then d += g dt^2; in place; returns status[4]."""
    assert x.dtype == np.float32 and d.dtype == np.float32 and x.flags.c_contiguous and d.flags.c_contiguous
    g = np.zeros(3, dtype=np.float32)
    g[:dim] = np.asarray(gravity, dtype=np.float32)[:dim]
    status = np.zeros(4, dtype=np.uint32)
    lib().oracle_pbmpm_integrate(dim, n, x.shape[-1], _p(x, F32P), _p(d, F32P), ct.c_float(dt), _p(g, F32P),
                                 _p(status, U32P))
    return status


def pbmpm_substep(dim: int, n: int, frac_bits: int, state: dict, ranges, iterations: int, relax: float,
                  polar_iters: int, band: int, dt: float, gravity):
    """One PB-MPM substep of the oracle on state = {x, v (the displacement d),
    C (the displacement gradient D), m, F}, updated in place.  Returns
    (the P2G grid of the last iteration, status[4] summed)."""
    status = np.zeros(4, dtype=np.int64)
    grid = None
    for _ in range(iterations):
        status += pbmpm_project_elastic(dim, state["F"], state["C"], relax, polar_iters)
        grid, st = p2g_quadratic(dim, n, frac_bits, state, ranges)
        status += st
        dg = pbmpm_grid_update(dim, n, grid.copy(), band)
        status += g2p(dim, n, dg, state, 0.0)
    status += pbmpm_integrate(dim, n, state["x"], state["v"], dt, gravity)
    update_F(dim, state["C"], state["F"], 1.0)
    return grid, status

