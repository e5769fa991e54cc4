"""ctypes binding of libmpm: the C entry points under the same names.

Argument marshalling only: device tensors are passed as raw pointers and the
current torch stream as the HIP stream; every step of the transfer runs in
the library's HIP kernels.  Loading fails loudly when libmpm.so is missing
(build it with ``python -m material_point_particle_amd.build``); there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes as ct
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmpm.so")

MPM_OK = 0
MPM_ERR_INVALID = -1
MPM_ERR_OVERFLOW = -2
MPM_ERR_DOMAIN = -3
MPM_ERR_WORKSPACE = -4
MPM_ERR_HIP = -6
MPM_ERR_SCRATCH = -7
# bytes of the static device scratch of mpm_p2g_isplit_noalloc (include/mpm.h)
MPM_ISPLIT_SCRATCH_BYTES = 256 * 1024 * 1024


class MpmError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {mpm_strerror(code)} (code {code})")
        self.code = code


class mpm_grid_desc(ct.Structure):
    _fields_ = [("dim", ct.c_int32), ("n", ct.c_int32), ("frac_bits", ct.c_int32), ("tile", ct.c_int32)]


class mpm_particles(ct.Structure):
    _fields_ = [("n", ct.c_int64), ("x", ct.c_void_p), ("v", ct.c_void_p), ("C", ct.c_void_p), ("m", ct.c_void_p)]


class mpm_ranges(ct.Structure):
    _fields_ = [("max_mass", ct.c_double), ("max_speed", ct.c_double), ("max_affine", ct.c_double)]


class mpm_ws_layout(ct.Structure):
    _fields_ = [(name, ct.c_size_t) for name in ("tile_count", "tile_start", "tile_active", "meta", "items", "rank",
                                                  "slot", "cell_key", "sorted", "scan_tmp")]
    _fields_ += [(name, ct.c_int64) for name in ("n_cells", "n_tiles", "max_items", "n_fields", "rows_per_item")]
    _fields_ += [("total_bytes", ct.c_size_t)]


EXPORTS = ("mpm_version", "mpm_strerror", "mpm_check_bounds", "mpm_workspace_bytes", "mpm_workspace_layout",
           "mpm_bin_particles", "mpm_p2g", "mpm_p2g_cic_split", "mpm_p2g_isplit", "mpm_isplit_workspace_bytes",
           "mpm_grid_update", "mpm_grid_clear", "mpm_g2p", "mpm_neohookean_affine", "mpm_update_deformation",
           "mpm_bin_resident", "mpm_g2p2g", "mpm_grid_clear_tiles", "mpm_gather_records",
           "mpm_p2g_isplit_noalloc", "mpm_pbmpm_project_elastic", "mpm_pbmpm_grid_update", "mpm_pbmpm_integrate",
           "mpm_grid_update_tiles", "mpm_g2p_records", "mpm_update_deformation_stress",
           "mpm_pbmpm_g2p_project", "mpm_pbmpm_g2p_project_records", "mpm_g2p_update_deformation_stress",
           "mpm_pbmpm_g2p_integrate")

_lib = None


def lib() -> ct.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmpm.so not found at {LIB_PATH}; build it with "
                               "`python -m material_point_particle_amd.build` (no CPU fallback exists)")
        L = ct.CDLL(LIB_PATH)
        P = ct.POINTER
        L.mpm_version.restype = ct.c_char_p
        L.mpm_version.argtypes = []
        L.mpm_strerror.restype = ct.c_char_p
        L.mpm_strerror.argtypes = [ct.c_int]
        L.mpm_check_bounds.restype = ct.c_int
        L.mpm_check_bounds.argtypes = [P(mpm_grid_desc), ct.c_int64, P(mpm_ranges), P(ct.c_double)]
        L.mpm_workspace_bytes.restype = ct.c_int
        L.mpm_workspace_bytes.argtypes = [P(mpm_grid_desc), ct.c_int64, P(ct.c_size_t)]
        L.mpm_workspace_layout.restype = ct.c_int
        L.mpm_workspace_layout.argtypes = [P(mpm_grid_desc), ct.c_int64, P(mpm_ws_layout)]
        L.mpm_bin_particles.restype = ct.c_int
        L.mpm_bin_particles.argtypes = [P(mpm_grid_desc), P(mpm_particles), P(mpm_ranges), ct.c_void_p, ct.c_size_t,
                                        ct.c_void_p, ct.c_void_p]
        L.mpm_p2g.restype = ct.c_int
        L.mpm_p2g.argtypes = [P(mpm_grid_desc), P(mpm_particles), P(mpm_ranges), ct.c_void_p, ct.c_size_t,
                              ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_p2g_cic_split.restype = ct.c_int
        L.mpm_p2g_cic_split.argtypes = [ct.c_int64, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int32,
                                        ct.c_int64, ct.c_int64, ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_p2g_isplit.restype = ct.c_int
        L.mpm_p2g_isplit.argtypes = [ct.c_int32, ct.c_int32, ct.c_int64, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                     ct.c_void_p, ct.c_void_p, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_void_p,
                                     ct.c_size_t, ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_p2g_isplit_noalloc.restype = ct.c_int
        L.mpm_p2g_isplit_noalloc.argtypes = [ct.c_int32, ct.c_int32, ct.c_int64, ct.c_void_p, ct.c_void_p,
                                             ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int64, ct.c_int64,
                                             ct.c_int64, ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_isplit_workspace_bytes.restype = ct.c_int
        L.mpm_isplit_workspace_bytes.argtypes = [ct.c_int32, ct.c_int32, ct.c_int64, P(ct.c_size_t)]
        L.mpm_grid_update.restype = ct.c_int
        L.mpm_grid_update.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                      ct.c_float, P(ct.c_float), ct.c_int32, ct.c_void_p]
        L.mpm_grid_clear.restype = ct.c_int
        L.mpm_grid_clear.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p]
        L.mpm_g2p.restype = ct.c_int
        L.mpm_g2p.argtypes = [P(mpm_grid_desc), ct.c_void_p, P(mpm_particles), ct.c_float, ct.c_void_p, ct.c_void_p]
        L.mpm_neohookean_affine.restype = ct.c_int
        L.mpm_neohookean_affine.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_void_p, ct.c_void_p, ct.c_float,
                                            ct.c_float, ct.c_float, ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_update_deformation.restype = ct.c_int
        L.mpm_update_deformation.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_void_p, ct.c_float, ct.c_void_p]
        L.mpm_update_deformation_stress.restype = ct.c_int
        L.mpm_update_deformation_stress.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_void_p, ct.c_void_p,
                                                    ct.c_float, ct.c_float, ct.c_float, ct.c_void_p, ct.c_void_p,
                                                    ct.c_void_p]
        L.mpm_bin_resident.restype = ct.c_int
        L.mpm_bin_resident.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_void_p, ct.c_size_t, ct.c_void_p,
                                       ct.c_void_p]
        L.mpm_g2p2g.restype = ct.c_int
        L.mpm_g2p2g.argtypes = [P(mpm_grid_desc), P(mpm_ranges), ct.c_void_p, ct.c_size_t, ct.c_int64, ct.c_void_p,
                                ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_float, P(ct.c_float),
                                ct.c_int32, ct.c_void_p, ct.c_void_p]
        L.mpm_grid_clear_tiles.restype = ct.c_int
        L.mpm_grid_clear_tiles.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_void_p, ct.c_void_p]
        L.mpm_pbmpm_g2p_project.restype = ct.c_int
        L.mpm_pbmpm_g2p_project.argtypes = [P(mpm_grid_desc), ct.c_void_p, P(mpm_particles), ct.c_void_p, ct.c_float,
                                            ct.c_int32, ct.c_void_p, ct.c_void_p]
        L.mpm_g2p_update_deformation_stress.restype = ct.c_int
        L.mpm_g2p_update_deformation_stress.argtypes = [P(mpm_grid_desc), ct.c_void_p, P(mpm_particles), ct.c_float,
                                                        ct.c_void_p, ct.c_void_p, ct.c_float, ct.c_float, ct.c_void_p,
                                                        ct.c_void_p, ct.c_void_p]
        L.mpm_pbmpm_g2p_integrate.restype = ct.c_int
        L.mpm_pbmpm_g2p_integrate.argtypes = [P(mpm_grid_desc), ct.c_void_p, P(mpm_particles), ct.c_void_p, ct.c_float,
                                              P(ct.c_float), ct.c_void_p, ct.c_void_p]
        L.mpm_pbmpm_g2p_project_records.restype = ct.c_int
        L.mpm_pbmpm_g2p_project_records.argtypes = [P(mpm_grid_desc), ct.c_void_p, P(mpm_particles), ct.c_void_p,
                                                    ct.c_float, ct.c_int32, P(mpm_ranges), ct.c_void_p, ct.c_size_t,
                                                    ct.c_void_p, ct.c_void_p]
        L.mpm_pbmpm_project_elastic.restype = ct.c_int
        L.mpm_pbmpm_project_elastic.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_void_p, ct.c_float, ct.c_int32,
                                                ct.c_void_p, ct.c_void_p]
        L.mpm_pbmpm_grid_update.restype = ct.c_int
        L.mpm_pbmpm_grid_update.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                            ct.c_int32, ct.c_void_p]
        L.mpm_pbmpm_integrate.restype = ct.c_int
        L.mpm_pbmpm_integrate.argtypes = [P(mpm_grid_desc), P(mpm_particles), ct.c_float, P(ct.c_float), ct.c_void_p,
                                          ct.c_void_p]
        L.mpm_grid_update_tiles.restype = ct.c_int
        L.mpm_grid_update_tiles.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_float,
                                            P(ct.c_float), ct.c_int32, ct.c_void_p]
        L.mpm_g2p_records.restype = ct.c_int
        L.mpm_g2p_records.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_size_t, ct.c_int64, ct.c_void_p, ct.c_float,
                                      ct.c_void_p, ct.c_void_p]
        L.mpm_gather_records.restype = ct.c_int
        L.mpm_gather_records.argtypes = [P(mpm_grid_desc), ct.c_void_p, ct.c_size_t, P(mpm_particles), ct.c_void_p,
                                         ct.c_void_p]
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != MPM_OK:
        raise MpmError(rc, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def grid_desc(dim: int, n: int, frac_bits: int, tile: int = 4) -> mpm_grid_desc:
    return mpm_grid_desc(dim, n, frac_bits, tile)


def ranges(max_mass: float, max_speed: float, max_affine: float) -> mpm_ranges:
    return mpm_ranges(max_mass, max_speed, max_affine)


def particles(n: int, x=None, v=None, C=None, m=None) -> mpm_particles:
    """Descriptor of component-major device tensors x[dim][n], v[dim][n],
    C[dim*dim][n], m[n] (float32, contiguous)."""
    for t in (x, v, C, m):
        if t is not None:
            assert t.is_contiguous() and t.dtype.itemsize == 4, "particle arrays must be contiguous float32"
    return mpm_particles(n, _ptr(x), _ptr(v), _ptr(C), _ptr(m))


# ------------------------------------------------------------------ entry points

def mpm_version() -> str:
    return lib().mpm_version().decode()


def mpm_strerror(code: int) -> str:
    try:
        return lib().mpm_strerror(code).decode()
    except RuntimeError:
        return f"error {code}"


def mpm_check_bounds(desc: mpm_grid_desc, n_particles: int, rng: mpm_ranges) -> float:
    """Returns log2 of the bound; raises MpmError(MPM_ERR_OVERFLOW) when refused."""
    out = ct.c_double(0.0)
    _check(lib().mpm_check_bounds(ct.byref(desc), n_particles, ct.byref(rng), ct.byref(out)), "mpm_check_bounds")
    return out.value


def mpm_workspace_bytes(desc: mpm_grid_desc, n_particles: int) -> int:
    out = ct.c_size_t(0)
    _check(lib().mpm_workspace_bytes(ct.byref(desc), n_particles, ct.byref(out)), "mpm_workspace_bytes")
    return out.value


def mpm_workspace_layout(desc: mpm_grid_desc, n_particles: int) -> mpm_ws_layout:
    out = mpm_ws_layout()
    _check(lib().mpm_workspace_layout(ct.byref(desc), n_particles, ct.byref(out)), "mpm_workspace_layout")
    return out


def mpm_bin_particles(desc, parts: mpm_particles, rng: mpm_ranges, ws, status, stream=None) -> None:
    _check(lib().mpm_bin_particles(ct.byref(desc), ct.byref(parts), ct.byref(rng), _ptr(ws), ws.numel() * ws.element_size(),
                                   _ptr(status), _stream(stream)), "mpm_bin_particles")


def mpm_p2g(desc, parts: mpm_particles, rng: mpm_ranges, bins, grid, status, stream=None) -> None:
    _check(lib().mpm_p2g(ct.byref(desc), ct.byref(parts), ct.byref(rng), _ptr(bins), _nbytes(bins), _ptr(grid),
                         _ptr(status), _stream(stream)), "mpm_p2g")


def mpm_p2g_cic_split(X, m, vel, order, cells: int, max_mass: int, max_speed: int, grid, status, stream=None) -> None:
    _check(lib().mpm_p2g_cic_split(m.numel(), _ptr(X), _ptr(m), _ptr(vel), _ptr(order), cells, max_mass, max_speed,
                                   _ptr(grid), _ptr(status), _stream(stream)), "mpm_p2g_cic_split")


def mpm_isplit_workspace_bytes(dim: int, n: int, np_: int) -> int:
    b = ct.c_size_t(0)
    _check(lib().mpm_isplit_workspace_bytes(dim, n, np_, ct.byref(b)), "mpm_isplit_workspace_bytes")
    return b.value


def mpm_p2g_isplit(dim: int, n: int, X, m, v, C, order, max_mass: int, max_speed: int, max_affine: int, grid,
                   status, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mpm_p2g_isplit(dim, n, m.numel(), _ptr(X), _ptr(m), _ptr(v), _ptr(C), _ptr(order), max_mass,
                                max_speed, max_affine, _ptr(workspace), ws_bytes, _ptr(grid), _ptr(status),
                                _stream(stream)), "mpm_p2g_isplit")


def mpm_p2g_isplit_noalloc(dim: int, n: int, X, m, v, C, order, max_mass: int, max_speed: int, max_affine: int,
                           grid, status, stream=None) -> None:
    """mpm_p2g_isplit's tiled path on the library's static device scratch
    (no allocation by the library or by this wrapper)."""
    _check(lib().mpm_p2g_isplit_noalloc(dim, n, m.numel(), _ptr(X), _ptr(m), _ptr(v), _ptr(C), _ptr(order), max_mass,
                                        max_speed, max_affine, _ptr(grid), _ptr(status), _stream(stream)),
           "mpm_p2g_isplit_noalloc")


def mpm_bin_resident(desc, parts: mpm_particles, ws, status, stream=None) -> None:
    _check(lib().mpm_bin_resident(ct.byref(desc), ct.byref(parts), _ptr(ws), ws.numel() * ws.element_size(),
                                  _ptr(status), _stream(stream)), "mpm_bin_resident")


def mpm_g2p2g(desc, rng: mpm_ranges, ws, n_particles: int, grid_in, grid_out, tiles_out, dt: float, gravity,
              sticky: int, status, stream=None, grid_clear=None, tiles_clear=None) -> None:
    g = (ct.c_float * 3)(*(list(gravity) + [0.0] * (3 - len(gravity))))
    _check(lib().mpm_g2p2g(ct.byref(desc), ct.byref(rng), _ptr(ws), _nbytes(ws), n_particles, _ptr(grid_in),
                           _ptr(grid_out),
                           _ptr(tiles_out), _ptr(grid_clear), _ptr(tiles_clear), dt, g, sticky, _ptr(status),
                           _stream(stream)), "mpm_g2p2g")


def mpm_grid_clear_tiles(desc, grid, tiles, stream=None) -> None:
    _check(lib().mpm_grid_clear_tiles(ct.byref(desc), _ptr(grid), _ptr(tiles), _stream(stream)),
           "mpm_grid_clear_tiles")


def mpm_grid_update_tiles(desc, grid, tiles, vg, dt: float, gravity, sticky: int, stream=None) -> None:
    g = (ct.c_float * 3)(*(list(gravity) + [0.0] * (3 - len(gravity))))
    _check(lib().mpm_grid_update_tiles(ct.byref(desc), _ptr(grid), _ptr(tiles), _ptr(vg), dt, g, sticky,
                                       _stream(stream)), "mpm_grid_update_tiles")


def mpm_g2p_records(desc, ws, n_particles: int, vg, dt: float, status, stream=None) -> None:
    _check(lib().mpm_g2p_records(ct.byref(desc), _ptr(ws), _nbytes(ws), n_particles, _ptr(vg), dt, _ptr(status),
                                 _stream(stream)), "mpm_g2p_records")


def mpm_gather_records(desc, ws, parts: mpm_particles, status, stream=None) -> None:
    _check(lib().mpm_gather_records(ct.byref(desc), _ptr(ws), _nbytes(ws), ct.byref(parts), _ptr(status),
                                    _stream(stream)), "mpm_gather_records")


def mpm_grid_update(desc, bins, grid, vg, dt: float, gravity, sticky: int, stream=None) -> None:
    g = (ct.c_float * 3)(*(list(gravity) + [0.0] * (3 - len(gravity))))
    _check(lib().mpm_grid_update(ct.byref(desc), _ptr(bins), _nbytes(bins), _ptr(grid), _ptr(vg), dt, g, sticky,
                                 _stream(stream)), "mpm_grid_update")


def mpm_grid_clear(desc, bins, grid, stream=None) -> None:
    _check(lib().mpm_grid_clear(ct.byref(desc), _ptr(bins), _nbytes(bins), _ptr(grid), _stream(stream)),
           "mpm_grid_clear")


def mpm_g2p(desc, vg, parts: mpm_particles, dt: float, status, stream=None) -> None:
    _check(lib().mpm_g2p(ct.byref(desc), _ptr(vg), ct.byref(parts), dt, _ptr(status), _stream(stream)), "mpm_g2p")


def mpm_neohookean_affine(desc, parts: mpm_particles, F, vol0, dt: float, mu: float, lam: float, C_out, status,
                          stream=None) -> None:
    _check(lib().mpm_neohookean_affine(ct.byref(desc), ct.byref(parts), _ptr(F), _ptr(vol0), dt, mu, lam, _ptr(C_out),
                                       _ptr(status), _stream(stream)), "mpm_neohookean_affine")


def mpm_update_deformation(desc, parts: mpm_particles, F, dt: float, stream=None) -> None:
    _check(lib().mpm_update_deformation(ct.byref(desc), ct.byref(parts), _ptr(F), dt, _stream(stream)),
           "mpm_update_deformation")


def mpm_update_deformation_stress(desc, parts: mpm_particles, F, vol0, dt: float, mu: float, lam: float, C_out,
                                  status, stream=None) -> None:
    _check(lib().mpm_update_deformation_stress(ct.byref(desc), ct.byref(parts), _ptr(F), _ptr(vol0), dt, mu, lam,
                                               _ptr(C_out), _ptr(status), _stream(stream)),
           "mpm_update_deformation_stress")


def mpm_pbmpm_g2p_project(desc, dg, parts: mpm_particles, F, relax: float, polar_iters: int, status,
                          stream=None) -> None:
    _check(lib().mpm_pbmpm_g2p_project(ct.byref(desc), _ptr(dg), ct.byref(parts), _ptr(F), relax, polar_iters,
                                       _ptr(status), _stream(stream)), "mpm_pbmpm_g2p_project")


def mpm_g2p_update_deformation_stress(desc, vg, parts: mpm_particles, dt: float, F, vol0, mu: float, lam: float,
                                      C_out, status, stream=None) -> None:
    _check(lib().mpm_g2p_update_deformation_stress(ct.byref(desc), _ptr(vg), ct.byref(parts), dt, _ptr(F), _ptr(vol0),
                                                   mu, lam, _ptr(C_out), _ptr(status), _stream(stream)),
           "mpm_g2p_update_deformation_stress")


def mpm_pbmpm_g2p_project_records(desc, dg, parts: mpm_particles, F, relax: float, polar_iters: int,
                                  rng: mpm_ranges, ws, status, stream=None) -> None:
    _check(lib().mpm_pbmpm_g2p_project_records(ct.byref(desc), _ptr(dg), ct.byref(parts), _ptr(F), relax,
                                               polar_iters, ct.byref(rng), _ptr(ws), _nbytes(ws), _ptr(status),
                                               _stream(stream)), "mpm_pbmpm_g2p_project_records")


def mpm_pbmpm_g2p_integrate(desc, dg, parts: mpm_particles, F, dt: float, gravity, status, stream=None) -> None:
    g = (ct.c_float * 3)(*(list(gravity) + [0.0] * (3 - len(gravity))))
    _check(lib().mpm_pbmpm_g2p_integrate(ct.byref(desc), _ptr(dg), ct.byref(parts), _ptr(F), dt, g, _ptr(status),
                                         _stream(stream)), "mpm_pbmpm_g2p_integrate")


def mpm_pbmpm_project_elastic(desc, parts: mpm_particles, F, relax: float, polar_iters: int, status,
                              stream=None) -> None:
    _check(lib().mpm_pbmpm_project_elastic(ct.byref(desc), ct.byref(parts), _ptr(F), relax, polar_iters, _ptr(status),
                                           _stream(stream)), "mpm_pbmpm_project_elastic")


def mpm_pbmpm_grid_update(desc, bins, grid, dg, band: int, stream=None) -> None:
    _check(lib().mpm_pbmpm_grid_update(ct.byref(desc), _ptr(bins), _nbytes(bins), _ptr(grid), _ptr(dg), band,
                                       _stream(stream)), "mpm_pbmpm_grid_update")


def mpm_pbmpm_integrate(desc, parts: mpm_particles, dt: float, gravity, status, stream=None) -> None:
    g = (ct.c_float * 3)(*(list(gravity) + [0.0] * (3 - len(gravity))))
    _check(lib().mpm_pbmpm_integrate(ct.byref(desc), ct.byref(parts), dt, g, _ptr(status), _stream(stream)),
           "mpm_pbmpm_integrate")

