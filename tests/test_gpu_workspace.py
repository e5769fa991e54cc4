"""Workspaces handed to the wrong call, through the C ABI.  The binning
stamps its workspace with the grid, the particle count, the declared ranges
and whether it is the checked or the resident binning; every kernel that
reads the bins compares the stamp with its own arguments before reading
anything else.  A mismatch adds and copies nothing and is counted once in
status[3]; the restricted grid update and clear fall back to every node, which
gives the dense pass's results.  (Workspaces too small for the call's own
grid and count are refused on the host: tests/test_abi_host.py.)
"""
import sys

import numpy as np
import pytest
import torch

from mpm_inputs import WORKLOADS, build, scaled

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mpm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import material_point_particle_amd as M
    M.lib()
    return M


def status_of(tr):
    return tr.status.cpu().numpy().view(np.uint32).tolist()


def test_p2g_refuses_bins_of_another_binning(mpm, oracle_lib):
    import material_point_particle_amd._lib as L
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    w = scaled(WORKLOADS["blobs_3d_256"], 1 << 14)
    host = build(w)
    rng = (w.max_mass, w.max_speed, w.max_affine)
    parts = DeviceParticles(host)
    tr = Transfer(w.dim, w.n, w.frac_bits, rng, parts.n)
    tr.bin(parts)
    say("stamp: P2G with other ranges, another count, resident bins")
    # other declared ranges than the binning's
    L.mpm_p2g(tr.desc, parts.desc(), L.ranges(rng[0], rng[1] * 2, rng[2]), tr.ws, tr.grid, tr.status)
    torch.cuda.synchronize()
    assert int(tr.grid.abs().sum()) == 0 and status_of(tr) == [0, 0, 0, 1]
    # another particle count (the workspace is large enough for it)
    fewer = L.particles(parts.n - 1, parts.x, parts.v, parts.C, parts.m)
    L.mpm_p2g(tr.desc, fewer, tr.ranges, tr.ws, tr.grid, tr.status)
    torch.cuda.synchronize()
    assert int(tr.grid.abs().sum()) == 0 and status_of(tr) == [0, 0, 0, 2]
    # the matching call deposits the oracle's grid
    tr.p2g(parts, binned=True)
    ref, _ = oracle_lib.p2g_quadratic(w.dim, w.n, w.frac_bits, host, rng)
    torch.cuda.synchronize()
    assert np.array_equal(tr.grid.cpu().numpy(), ref) and status_of(tr) == [0, 0, 0, 2]
    # bins of the resident binning (records not range-checked): refused by P2G
    tr.grid.zero_()
    L.mpm_bin_resident(tr.desc, parts.desc(), tr.ws, tr.status)
    tr.p2g(parts, binned=True)
    torch.cuda.synchronize()
    assert int(tr.grid.abs().sum()) == 0 and status_of(tr) == [0, 0, 0, 3]


def test_fused_and_gather_refuse_another_count(mpm):
    import material_point_particle_amd._lib as L
    from material_point_particle_amd.transfer import DeviceParticles, ResidentSubsteps, Transfer
    w = scaled(WORKLOADS["dam_3d_256"], 1 << 14, n=64)
    host = build(w)
    ex = w.extra
    parts = DeviceParticles(host)
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    rs = ResidentSubsteps(tr, parts, ex["dt"], ex["gravity"], ex["sticky"])
    rs.start()
    torch.cuda.synchronize()
    assert status_of(tr) == [0, 0, 0, 0]
    say("stamp: fused substep and gather with another count")
    x0 = parts.x.clone()
    out = torch.zeros_like(tr.grid)
    tiles = torch.zeros_like(rs.tiles[0])
    L.mpm_g2p2g(tr.desc, tr.ranges, tr.ws, parts.n - 1, rs.grid, out, tiles, ex["dt"], ex["gravity"], ex["sticky"],
                tr.status)
    fewer = L.particles(parts.n - 1, parts.x, parts.v, parts.C, parts.m)
    L.mpm_gather_records(tr.desc, tr.ws, fewer, tr.status)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0 and int(tiles.sum()) == 0
    assert torch.equal(parts.x, x0)
    assert status_of(tr) == [0, 0, 0, 2]


def test_restricted_update_with_bins_of_another_grid_updates_every_node(mpm, oracle_lib):
    """Bins of a 64^3 binning handed to the update of a 32^3 grid: every node is
    updated (the dense pass), and the restricted clear zeroes every node."""
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    w64 = scaled(WORKLOADS["dam_3d_256"], 1 << 14, n=64)
    parts = DeviceParticles(build(w64))
    tr64 = Transfer(3, 64, w64.frac_bits, (w64.max_mass, w64.max_speed, w64.max_affine), parts.n)
    tr64.bin(parts)
    w32 = scaled(WORKLOADS["dam_3d_256"], 1 << 12, n=32)
    h32 = build(w32)
    ex = w32.extra
    grid, _ = oracle_lib.p2g_quadratic(3, 32, w32.frac_bits, h32, (w32.max_mass, w32.max_speed, w32.max_affine))
    vg_ref = oracle_lib.grid_update(3, 32, grid.copy(), ex["dt"], ex["gravity"], ex["sticky"])
    tr32 = Transfer(3, 32, w32.frac_bits, (w32.max_mass, w32.max_speed, w32.max_affine), w32.n_particles)
    tr32.ws = tr64.ws                       # the 64^3 binning's workspace, larger than 32^3 needs
    tr32.grid.copy_(torch.from_numpy(grid))
    tr32.vg.fill_(7.0)
    say("stamp: restricted update and clear with another grid's bins")
    tr32.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
    torch.cuda.synchronize()
    assert np.array_equal(tr32.vg.cpu().numpy(), vg_ref)
    assert int(tr32.grid.abs().sum()) == 0
    tr32.grid.fill_(5)
    tr32.clear(active=True)
    torch.cuda.synchronize()
    assert int(tr32.grid.abs().sum()) == 0
