"""Host-only checks of the C ABI: the library loads, exports every entry point
include/mpm.h declares, and its host-side logic (bounds line, workspace
layout, argument validation) behaves as documented.  No kernel is launched:
every call here returns before touching the device."""
import ctypes as ct
import math
import os
import re

import pytest

import material_point_particle_amd as M
from material_point_particle_amd import _lib as L
from mpm_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "mpm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = declared_entry_points()
    assert set(names) == set(L.EXPORTS), names
    lib = M.lib()
    for name in names:
        assert hasattr(lib, name), name
        assert ct.cast(getattr(lib, name), ct.c_void_p).value
        # and the package's binding carries a wrapper of the same name
        assert callable(getattr(M, name, None)), name


def test_version_and_errors():
    assert "gfx950" in M.mpm_version()
    for code in (0, -1, -2, -3, -4, -6):
        assert M.mpm_strerror(code)
    assert "unknown" in M.mpm_strerror(12345)


@pytest.mark.parametrize("name", ["pile_2d", "dam_3d_128", "blobs_3d_256", "dam_3d_256"])
def test_bounds_accept_the_workloads_and_agree_with_the_oracle(oracle_lib, name):
    w = WORKLOADS[name]
    r = (w.max_mass, w.max_speed, w.max_affine)
    lb = M.mpm_check_bounds(M.grid_desc(w.dim, w.n, w.frac_bits), w.n_particles, M.ranges(*r))
    assert lb < 63
    assert math.isclose(lb, oracle_lib.p2g_log2_bound(w.dim, w.n, w.frac_bits, w.n_particles, r), abs_tol=1e-3)


def test_bounds_refuse_overflowing_ranges():
    with pytest.raises(M.MpmError) as e:
        M.mpm_check_bounds(M.grid_desc(3, 256, 40), 1 << 24, M.ranges(2.0, 8.0, 0.5))
    assert e.value.code == L.MPM_ERR_OVERFLOW
    # one work item of 2048 particles must stay below 2^53 on chip
    with pytest.raises(M.MpmError):
        M.mpm_check_bounds(M.grid_desc(3, 64, 50), 1, M.ranges(1.0, 1.0, 0.0))


def test_descriptor_validation():
    r = M.ranges(1.0, 1.0, 1.0)
    for bad in [(4, 64, 32), (3, 100, 32), (3, 4, 32), (3, 1024, 32), (2, 64, 61), (2, 64, -1)]:
        with pytest.raises(M.MpmError) as e:
            M.mpm_check_bounds(M.grid_desc(*bad), 10, r)
        assert e.value.code == L.MPM_ERR_INVALID
    with pytest.raises(M.MpmError):
        M.mpm_check_bounds(M.grid_desc(3, 64, 32, tile=8), 10, r)
    with pytest.raises(M.MpmError):
        M.mpm_check_bounds(M.grid_desc(3, 64, 32), 10, M.ranges(float("nan"), 1.0, 1.0))


def test_workspace_layout_is_disjoint_and_aligned():
    for dim, n, N in [(2, 64, 3500), (3, 128, 1 << 20), (3, 256, 1 << 24), (3, 8, 0), (2, 8, 1)]:
        d = M.grid_desc(dim, n, 20)
        lay = M.mpm_workspace_layout(d, N)
        assert M.mpm_workspace_bytes(d, N) == lay.total_bytes
        assert lay.n_cells == n ** dim and lay.n_tiles == (n // 4) ** dim
        assert lay.n_fields == {2: 12, 3: 16}[dim]     # x, v, C, m padded to a multiple of 4 floats
        spans = sorted([
            (lay.tile_count, 4 * lay.n_tiles), (lay.tile_start, 4 * (lay.n_tiles + 1)), (lay.tile_active, lay.n_tiles),
            (lay.meta, 128), (lay.items, 16 * lay.max_items), (lay.rank, 4 * max(N, 1)), (lay.slot, 4 * max(N, 1)),
            (lay.cell_key, max(N, 1) + 4), (lay.sorted, 4 * lay.n_fields * max(N, 1)),
            (lay.scan_tmp, 4 * (2 + lay.rows_per_item) * ((lay.n_tiles + 4095) // 4096))])
        for (a, la), (b, _) in zip(spans, spans[1:]):
            assert a % 256 == 0 and a + la <= b
        assert spans[-1][0] + spans[-1][1] <= lay.total_bytes


def test_isplit_workspace_size():
    # tile counters and starts (8^dim-cell tiles over the n - 2 base nodes per
    # axis; up to 8 counters per tile, at most 2^22 in all), plus a rank and a
    # 128-byte record per visited particle, in 256-byte sections
    def r(b):
        return (b + 255) // 256 * 256
    for dim, n, N in [(3, 128, 1 << 20), (2, 64, 3500), (3, 10, 1), (2, 2048, 0), (3, 1024, 5), (2, 32767, 7)]:
        t = ((n - 2 + 7) // 8) ** dim
        slots = 8
        while slots > 1 and t * slots > 1 << 22:
            slots //= 2
        e = t * slots
        blocks = (e + 1023) // 1024
        want = r(4 * e) + r(8 * e) + r(8 * blocks) + r(16) + r(4 * max(N, 1)) + r(128 * max(N, 1))
        assert M.mpm_isplit_workspace_bytes(dim, n, N) == want
    with pytest.raises(M.MpmError):
        M.mpm_isplit_workspace_bytes(3, 2, 10)


def test_tile_arrays_sit_at_offsets_independent_of_the_particle_count():
    # mpm_grid_update finds tile_count and tile_active in a workspace without
    # knowing the particle count it was sized for
    for dim, n in [(2, 64), (3, 256)]:
        d = M.grid_desc(dim, n, 20)
        base = M.mpm_workspace_layout(d, 0)
        for N in (1, 3500, 1 << 20):
            lay = M.mpm_workspace_layout(d, N)
            assert (lay.tile_count, lay.tile_start, lay.tile_active, lay.meta) == (
                base.tile_count, base.tile_start, base.tile_active, base.meta)
            assert lay.meta < lay.items


def test_entry_points_reject_bad_arguments_before_any_launch():
    lib = M.lib()
    d = M.grid_desc(3, 64, 32)
    r = M.ranges(1.0, 1.0, 1.0)
    p = L.mpm_particles(10, None, None, None, None)
    status = ct.c_void_p(256)
    grid = ct.c_void_p(4096)
    assert lib.mpm_p2g(ct.byref(d), ct.byref(p), ct.byref(r), None, 0, grid, status, None) == L.MPM_ERR_INVALID
    assert lib.mpm_p2g(None, ct.byref(p), ct.byref(r), None, 0, grid, status, None) == L.MPM_ERR_INVALID
    misaligned = ct.c_void_p(4099)
    p2 = L.mpm_particles(10, 4096, 4096, 4096, 4096)
    assert lib.mpm_p2g(ct.byref(d), ct.byref(p2), ct.byref(r), None, 0, misaligned, status, None) == L.MPM_ERR_INVALID
    assert lib.mpm_bin_particles(ct.byref(d), ct.byref(p2), ct.byref(r), ct.c_void_p(4096), 16, status,
                                 None) == L.MPM_ERR_WORKSPACE
    assert lib.mpm_bin_particles(ct.byref(d), ct.byref(p2), ct.byref(r), ct.c_void_p(4100), 1 << 30, status,
                                 None) == L.MPM_ERR_INVALID
    big = L.mpm_ranges(1e30, 1e30, 1e30)
    assert lib.mpm_p2g(ct.byref(d), ct.byref(p2), ct.byref(big), None, 0, grid, status, None) == L.MPM_ERR_OVERFLOW
    # a workspace too small for this grid and particle count is refused before any launch
    need_bins = M.mpm_workspace_bytes(d, 10)
    wsp = ct.c_void_p(1 << 20)
    assert lib.mpm_p2g(ct.byref(d), ct.byref(p2), ct.byref(r), wsp, need_bins - 1, grid, status,
                       None) == L.MPM_ERR_WORKSPACE
    assert lib.mpm_p2g(ct.byref(d), ct.byref(p), ct.byref(r), ct.c_void_p((1 << 20) + 8), need_bins, grid, status,
                       None) == L.MPM_ERR_INVALID
    assert lib.mpm_p2g_cic_split(256, None, None, None, None, 8, 1000, 1000, grid, status, None) == L.MPM_ERR_INVALID
    assert lib.mpm_p2g_cic_split(1 << 40, 4096, 4096, 4096, None, 8, 1 << 20, 1 << 20, grid, status,
                                 None) == L.MPM_ERR_INVALID
    assert lib.mpm_p2g_cic_split(1 << 30, 4096, 4096, 4096, None, 8, 1 << 20, 1 << 20, grid, status,
                                 None) == L.MPM_ERR_OVERFLOW
    A = ct.c_void_p(4096)
    W = (ct.c_void_p(1 << 20), 1 << 30)

    def isplit(dim, n, np_, X, m, v, C, order, mm, ms, ma, ws=(None, 0)):
        return lib.mpm_p2g_isplit(dim, n, np_, X, m, v, C, order, mm, ms, ma, *ws, grid, status, None)
    assert isplit(3, 64, 10, None, A, A, A, None, 1000, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(3, 64, 10, A, ct.c_void_p(4100), A, A, None, 1000, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(4, 64, 10, A, A, A, A, None, 1000, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(3, 2, 10, A, A, A, A, None, 1000, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(3, 64, 10, A, A, A, A, None, -1, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(3, 64, 10, A, A, A, A, ct.c_void_p(4098), 1000, 1000, 1000) == L.MPM_ERR_INVALID
    assert isplit(3, 64, 1 << 30, A, A, A, A, None, 1 << 20, 1 << 20, 1 << 20) == L.MPM_ERR_OVERFLOW
    assert isplit(3, 64, 1, A, A, A, A, None, 1 << 40, 1 << 20, 1 << 20) == L.MPM_ERR_OVERFLOW
    assert isplit(3, 64, 10, A, A, A, A, None, 1000, 1000, 1000, (ct.c_void_p(4360), 1 << 30)) == L.MPM_ERR_INVALID
    need = M.mpm_isplit_workspace_bytes(3, 64, 10)
    assert isplit(3, 64, 10, A, A, A, A, None, 1000, 1000, 1000, (W[0], need - 1)) == L.MPM_ERR_WORKSPACE
    # resident substep entries
    g3 = (ct.c_float * 3)(0, -9.8, 0)
    T = ct.c_void_p(1 << 16)
    G3, T3 = ct.c_void_p(1 << 20), ct.c_void_p(1 << 17)

    def g2p2g(ws, grid_in, grid_out, tiles_out, grav=g3, sticky=2, rng=r, clear=(None, None), ws_bytes=1 << 30):
        return lib.mpm_g2p2g(ct.byref(d), ct.byref(rng), ct.c_void_p(ws), ws_bytes, 10, grid_in, grid_out, tiles_out,
                             clear[0], clear[1], 1e-4, grav, sticky, status, None)
    assert g2p2g(4096, None, grid, T, ws_bytes=need_bins - 1) == L.MPM_ERR_WORKSPACE
    assert g2p2g(4096, grid, grid, T) == L.MPM_ERR_INVALID                             # grid_in == grid_out
    assert g2p2g(4100, None, grid, T) == L.MPM_ERR_INVALID                             # misaligned workspace
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, sticky=100) == L.MPM_ERR_INVALID    # sticky beyond n/2
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, grav=None) == L.MPM_ERR_INVALID     # no gravity
    assert g2p2g(4096, None, grid, T, rng=M.ranges(1e30, 1e30, 1e30)) == L.MPM_ERR_OVERFLOW
    # the third grid: distinct from both others, its flags distinct from tiles_out, both aligned
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, clear=(grid, T3)) == L.MPM_ERR_INVALID
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, clear=(ct.c_void_p(8192), T3)) == L.MPM_ERR_INVALID
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, clear=(G3, T)) == L.MPM_ERR_INVALID
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, clear=(G3, None)) == L.MPM_ERR_INVALID
    assert g2p2g(4096, ct.c_void_p(8192), grid, T, clear=(ct.c_void_p((1 << 20) + 4), T3)) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_clear_tiles(ct.byref(d), ct.c_void_p(4100), T, None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_clear_tiles(None, grid, T, None) == L.MPM_ERR_INVALID
    # the split resident substep's entries
    VG = ct.c_void_p(1 << 21)
    assert lib.mpm_grid_update_tiles(ct.byref(d), grid, T, VG, 1e-4, g3, 100, None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update_tiles(ct.byref(d), grid, T, VG, 1e-4, None, 2, None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update_tiles(ct.byref(d), grid, ct.c_void_p((1 << 16) + 2), VG, 1e-4, g3, 2,
                                     None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update_tiles(ct.byref(d), grid, T, VG, -1.0, g3, 2, None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update_tiles(None, grid, T, VG, 1e-4, g3, 2, None) == L.MPM_ERR_INVALID
    assert lib.mpm_g2p_records(ct.byref(d), ct.c_void_p(4096), need_bins - 1, 10, VG, 1e-4, status,
                               None) == L.MPM_ERR_WORKSPACE
    assert lib.mpm_g2p_records(ct.byref(d), ct.c_void_p(4100), 1 << 30, 10, VG, 1e-4, status,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_g2p_records(ct.byref(d), ct.c_void_p(4096), 1 << 30, -1, VG, 1e-4, status,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_g2p_records(ct.byref(d), ct.c_void_p(4096), 1 << 30, 10, VG, float("nan"), status,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_gather_records(ct.byref(d), ct.c_void_p(4096), 1 << 30,
                                  ct.byref(L.mpm_particles(10, 4096, 4096, None, 4096)), status,
                                  None) == L.MPM_ERR_INVALID                           # no C
    assert lib.mpm_gather_records(ct.byref(d), ct.c_void_p(4096), need_bins - 1, ct.byref(p2), status,
                                  None) == L.MPM_ERR_WORKSPACE
    assert lib.mpm_bin_resident(ct.byref(d), ct.byref(p2), ct.c_void_p(4096), 16, status,
                                None) == L.MPM_ERR_WORKSPACE
    g = (ct.c_float * 3)(0, -9.8, 0)
    assert lib.mpm_grid_update(ct.byref(d), None, 0, grid, ct.c_void_p(4096), 1e-4, g, 100,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update(ct.byref(d), None, 0, grid, ct.c_void_p(4096), 1e-4, None, 2,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_update(ct.byref(d), ct.c_void_p(4100), 1 << 30, grid, ct.c_void_p(4096), 1e-4, g, 2,
                               None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_clear(ct.byref(d), None, 0, ct.c_void_p(4100), None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_clear(ct.byref(d), ct.c_void_p(4100), 1 << 30, grid, None) == L.MPM_ERR_INVALID
    assert lib.mpm_grid_clear(None, None, 0, grid, None) == L.MPM_ERR_INVALID
    # the restricted update and clear need the workspace's tile arrays and meta words
    lay0 = M.mpm_workspace_layout(d, 0)
    prefix = lay0.meta + 128
    assert lib.mpm_grid_update(ct.byref(d), wsp, prefix - 1, grid, ct.c_void_p(4096), 1e-4, g, 2,
                               None) == L.MPM_ERR_WORKSPACE
    assert lib.mpm_grid_clear(ct.byref(d), wsp, prefix - 1, grid, None) == L.MPM_ERR_WORKSPACE
    p3 = L.mpm_particles(10, 4096, 4096, None, 4096)
    assert lib.mpm_g2p(ct.byref(d), ct.c_void_p(4096), ct.byref(p3), 1e-4, status, None) == L.MPM_ERR_INVALID
    p4 = L.mpm_particles(10, 4096, 4096, 4096, 4096)
    ok = (ct.c_void_p(4096), ct.c_void_p(4096), 1e-4, 1e5, 1e5, ct.c_void_p(4096), status)
    assert lib.mpm_neohookean_affine(ct.byref(d), ct.byref(p3), *ok, None) == L.MPM_ERR_INVALID     # no C
    assert lib.mpm_neohookean_affine(ct.byref(d), ct.byref(p4), None, *ok[1:], None) == L.MPM_ERR_INVALID
    assert lib.mpm_neohookean_affine(ct.byref(d), ct.byref(p4), *ok[:3], -1.0, *ok[4:], None) == L.MPM_ERR_INVALID
    assert lib.mpm_neohookean_affine(ct.byref(d), ct.byref(p4), ct.c_void_p(4098), *ok[1:], None) == L.MPM_ERR_INVALID
    assert lib.mpm_neohookean_affine(None, ct.byref(p4), *ok, None) == L.MPM_ERR_INVALID
    assert lib.mpm_update_deformation(ct.byref(d), ct.byref(p3), ct.c_void_p(4096), 1e-4, None) == L.MPM_ERR_INVALID
    assert lib.mpm_update_deformation(ct.byref(d), ct.byref(p4), None, 1e-4, None) == L.MPM_ERR_INVALID
    # F, vol0, dt, mu, lambda, C_out, status: one fault per call
    okf = (ct.c_void_p(8192), ct.c_void_p(12288), 1e-4, 1e5, 1e5, ct.c_void_p(16384), status)
    fused = lib.mpm_update_deformation_stress
    assert fused(ct.byref(d), ct.byref(p3), *okf, None) == L.MPM_ERR_INVALID                       # no C
    assert fused(ct.byref(d), ct.byref(p4), None, *okf[1:], None) == L.MPM_ERR_INVALID             # no F
    assert fused(ct.byref(d), ct.byref(p4), ct.c_void_p(8194), *okf[1:], None) == L.MPM_ERR_INVALID
    assert fused(ct.byref(d), ct.byref(p4), *okf[:4], -1.0, *okf[5:], None) == L.MPM_ERR_INVALID
    assert fused(ct.byref(d), ct.byref(p4), *okf[:5], ct.c_void_p(4096), status, None) == L.MPM_ERR_INVALID  # C' = C
    assert fused(ct.byref(d), ct.byref(p4), *okf[:5], ct.c_void_p(8192), status, None) == L.MPM_ERR_INVALID  # C' = F
    assert fused(None, ct.byref(p4), *okf, None) == L.MPM_ERR_INVALID
    # G2P with the F update and stress in one launch: vg, particles, dt, F, vol0, mu, lambda, C_out, status
    g2s = lib.mpm_g2p_update_deformation_stress
    VG8 = ct.c_void_p(20480)
    ok2 = (ct.c_void_p(8192), ct.c_void_p(12288), 1e5, 1e5, ct.c_void_p(16384), status)
    assert g2s(ct.byref(d), VG8, ct.byref(p3), 1e-4, *ok2, None) == L.MPM_ERR_INVALID               # no C
    assert g2s(ct.byref(d), VG8, ct.byref(L.mpm_particles(10, 4096, 4096, 4096, None)), 1e-4, *ok2,
               None) == L.MPM_ERR_INVALID                                                        # no m
    assert g2s(ct.byref(d), None, ct.byref(p4), 1e-4, *ok2, None) == L.MPM_ERR_INVALID              # no vg
    assert g2s(ct.byref(d), VG8, ct.byref(p4), 1e-4, None, *ok2[1:], None) == L.MPM_ERR_INVALID     # no F
    assert g2s(ct.byref(d), VG8, ct.byref(p4), -1e-4, *ok2, None) == L.MPM_ERR_INVALID
    assert g2s(ct.byref(d), VG8, ct.byref(p4), 1e-4, *ok2[:2], -1.0, *ok2[3:], None) == L.MPM_ERR_INVALID
    assert g2s(ct.byref(d), VG8, ct.byref(p4), 1e-4, *ok2[:4], ct.c_void_p(4096), status,
               None) == L.MPM_ERR_INVALID                                                        # C' = C
    assert g2s(ct.byref(d), VG8, ct.byref(p4), 1e-4, *ok2[:4], ct.c_void_p(8192), status,
               None) == L.MPM_ERR_INVALID                                                        # C' = F
    assert g2s(None, VG8, ct.byref(p4), 1e-4, *ok2, None) == L.MPM_ERR_INVALID
    # PB-MPM gather with the next projection: dg, particles, F, relax, iterations, status
    gp = lib.mpm_pbmpm_g2p_project
    dg = ct.c_void_p(20480)
    assert gp(ct.byref(d), None, ct.byref(p4), ct.c_void_p(8192), 1.5, 12, status, None) == L.MPM_ERR_INVALID
    assert gp(ct.byref(d), dg, ct.byref(p3), ct.c_void_p(8192), 1.5, 12, status, None) == L.MPM_ERR_INVALID  # no C
    assert gp(ct.byref(d), dg, ct.byref(p4), None, 1.5, 12, status, None) == L.MPM_ERR_INVALID               # no F
    assert gp(ct.byref(d), dg, ct.byref(p4), ct.c_void_p(8192), 2.5, 12, status, None) == L.MPM_ERR_INVALID
    assert gp(ct.byref(d), dg, ct.byref(p4), ct.c_void_p(8192), 1.5, 65, status, None) == L.MPM_ERR_INVALID
    assert gp(None, dg, ct.byref(p4), ct.c_void_p(8192), 1.5, 12, status, None) == L.MPM_ERR_INVALID
    # the loop's last gather with the integrate step and the F update: dg, particles, F, dt, gravity, status
    gi = lib.mpm_pbmpm_g2p_integrate
    gv = (ct.c_float * 3)(0.0, -9.8, 0.0)
    assert gi(ct.byref(d), dg, ct.byref(p3), ct.c_void_p(8192), 1e-3, gv, status, None) == L.MPM_ERR_INVALID  # no C
    assert gi(ct.byref(d), dg, ct.byref(p4), None, 1e-3, gv, status, None) == L.MPM_ERR_INVALID             # no F
    assert gi(ct.byref(d), None, ct.byref(p4), ct.c_void_p(8192), 1e-3, gv, status, None) == L.MPM_ERR_INVALID
    assert gi(ct.byref(d), dg, ct.byref(p4), ct.c_void_p(8192), 1e-3, None, status, None) == L.MPM_ERR_INVALID
    assert gi(ct.byref(d), dg, ct.byref(p4), ct.c_void_p(8192), -1e-3, gv, status, None) == L.MPM_ERR_INVALID
    assert gi(None, dg, ct.byref(p4), ct.c_void_p(8192), 1e-3, gv, status, None) == L.MPM_ERR_INVALID
    # the same with the binned records rewritten: also ranges, masses and the binning's workspace
    gpr = lib.mpm_pbmpm_g2p_project_records
    F8 = ct.c_void_p(8192)
    wsr = (ct.byref(r), wsp, need_bins, status)
    nom = L.mpm_particles(10, 4096, 4096, 4096, None)
    assert gpr(ct.byref(d), dg, ct.byref(p3), F8, 1.5, 12, *wsr, None) == L.MPM_ERR_INVALID          # no C
    assert gpr(ct.byref(d), dg, ct.byref(nom), F8, 1.5, 12, *wsr, None) == L.MPM_ERR_INVALID         # no m
    assert gpr(ct.byref(d), dg, ct.byref(p4), None, 1.5, 12, *wsr, None) == L.MPM_ERR_INVALID        # no F
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 2.5, 12, *wsr, None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, -1, *wsr, None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, None, *wsr[1:], None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, ct.byref(L.mpm_ranges(-1.0, 1.0, 1.0)), *wsr[1:],
               None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, ct.byref(big), *wsr[1:], None) == L.MPM_ERR_OVERFLOW
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, ct.byref(r), None, need_bins, status,
               None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, ct.byref(r), ct.c_void_p((1 << 20) + 8), need_bins,
               status, None) == L.MPM_ERR_INVALID
    assert gpr(ct.byref(d), dg, ct.byref(p4), F8, 1.5, 12, ct.byref(r), wsp, need_bins - 1, status,
               None) == L.MPM_ERR_WORKSPACE


def test_noalloc_isplit_refuses_inputs_past_its_static_scratch():
    """mpm_p2g_isplit_noalloc checks the workspace its input needs against the
    static scratch before any device call; the pointers here are only aligned
    placeholders, never dereferenced."""
    lib = M.lib()
    fake = ct.c_void_p(1 << 20)
    np_ = 1 << 24
    assert M.mpm_isplit_workspace_bytes(3, 128, np_) > L.MPM_ISPLIT_SCRATCH_BYTES
    rc = lib.mpm_p2g_isplit_noalloc(3, 128, np_, fake, fake, fake, fake, None, 1, 1, 1, fake, fake, None)
    assert rc == L.MPM_ERR_SCRATCH
    assert "static scratch" in M.mpm_strerror(rc)
    # the bounds line and argument checks come first, as in mpm_p2g_isplit
    assert lib.mpm_p2g_isplit_noalloc(3, 128, np_, fake, fake, fake, fake, None, 1 << 40, 1 << 20, 1, fake, fake,
                                      None) == L.MPM_ERR_OVERFLOW
    assert lib.mpm_p2g_isplit_noalloc(4, 128, 10, fake, fake, fake, fake, None, 1, 1, 1, fake, fake,
                                      None) == L.MPM_ERR_INVALID
    # the largest 3D workload that fits: about 2M particles (132 bytes each) on 128^3
    assert M.mpm_isplit_workspace_bytes(3, 128, 2_000_000) <= L.MPM_ISPLIT_SCRATCH_BYTES
    assert M.mpm_isplit_workspace_bytes(3, 128, 2_100_000) > L.MPM_ISPLIT_SCRATCH_BYTES


def test_empty_calls_of_the_one_pass_entry_points_return_before_any_launch():
    """With no particles, the one-pass calls validate their descriptors and
    return MPM_OK without a device call (the pointers are aligned
    placeholders, never dereferenced), as the calls they combine do."""
    lib = M.lib()
    d = L.grid_desc(3, 32, 28)
    p0 = L.mpm_particles(0, None, None, None, None)
    fake = ct.c_void_p(4096)
    assert lib.mpm_update_deformation_stress(ct.byref(d), ct.byref(p0), None, None, 1e-4, 1e5, 1e5, None, fake,
                                             None) == L.MPM_OK
    assert lib.mpm_pbmpm_g2p_project(ct.byref(d), fake, ct.byref(p0), None, 1.5, 12, fake, None) == L.MPM_OK
    r = L.mpm_ranges(1.0, 1.0, 1.0)
    assert lib.mpm_pbmpm_g2p_project_records(ct.byref(d), fake, ct.byref(p0), None, 1.5, 12, ct.byref(r), fake,
                                             M.mpm_workspace_bytes(d, 0), fake, None) == L.MPM_OK
    assert lib.mpm_update_deformation(ct.byref(d), ct.byref(p0), None, 1e-4, None) == L.MPM_OK
    assert lib.mpm_g2p_update_deformation_stress(ct.byref(d), fake, ct.byref(p0), 1e-4, None, None, 1e5, 1e5, None,
                                                 fake, None) == L.MPM_OK
    assert lib.mpm_pbmpm_g2p_integrate(ct.byref(d), fake, ct.byref(p0), None, 1e-3,
                                       (ct.c_float * 3)(0.0, -9.8, 0.0), fake, None) == L.MPM_OK

