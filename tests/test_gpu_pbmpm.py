"""GPU parity of the position-based MPM (PB-MPM) iteration loop for an
elastic material against the oracle, through the C ABI: the elastic
projection (float64 Newton polar iteration, bit-exact), the displacement-form
grid update with the guardian (dense and restricted to reachable tiles), the
integrate step, and whole substeps of the jelly cube in lockstep with the
oracle's own trajectory (20 substeps of 5 iterations at 64^3; one substep of
the 8M-particle cube at 256^3): particle state, deformation gradient and the
last iteration's P2G grid bit for bit, status counters equal.
"""
import sys

import numpy as np
import pytest
import torch

from mpm_inputs import WORKLOADS, build
from mpm_inputs import generators as G

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def assert_same(a, b, what):
    """Bit for bit (the sign of a zero included)."""
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, what
    ab = a.view(np.uint32) if a.dtype == np.float32 else a
    bb = b.view(np.uint32) if b.dtype == np.float32 else b
    if not np.array_equal(ab, bb):
        diff = np.argwhere(ab != bb)
        i = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} entries differ; first at {i}: gpu {a[i]!r} oracle {b[i]!r}")


def random_deformations(seed, k, dim):
    """Deformation gradients near rotations times stretches and displacement
    gradients of moderate size, a few inverted ones among them."""
    u = G.uniform01(seed, 1, k * dim * dim).reshape(dim * dim, k)
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.4 * (u - 0.5)).astype(np.float32)
    v = G.uniform01(seed, 2, k * dim * dim).reshape(dim * dim, k)
    D = (0.3 * (v - 0.5)).astype(np.float32)
    D[:, :7] = 0.0
    D[0, :7] = -2.5                                   # (I + D) F inverted
    return np.ascontiguousarray(F), np.ascontiguousarray(D)


@pytest.mark.parametrize("dim", [2, 3])
def test_projection_bit_exact(mpm, oracle_lib, dim):
    from material_point_particle_amd import _lib as L
    k = 100_003
    F, D = random_deformations(0x9B + dim, k, dim)
    for relax, iters in ((1.5, 12), (1.0, 3), (0.5, 0)):
        ref = D.copy()
        rst = oracle_lib.pbmpm_project_elastic(dim, F, ref, relax, iters)
        Fd, Dd = dev(F), dev(D)
        st = torch.zeros(4, dtype=torch.int32, device="cuda")
        parts = L.particles(k, None, None, Dd, None)
        L.mpm_pbmpm_project_elastic(L.grid_desc(dim, 64, 32), parts, Fd, relax, iters, st)
        torch.cuda.synchronize()
        say("pbmpm projection", dim, relax, iters)
        assert_same(Dd.cpu().numpy(), ref, f"D after the projection ({dim}D, relax {relax}, {iters} Newton steps)")
        assert u32(st).tolist() == rst.tolist() and rst[0] >= 7


@pytest.mark.parametrize("dim", [2, 3])
def test_projection_wide_exponents_bit_exact(mpm, oracle_lib, dim):
    """The projection on deformation gradients whose entries span float32's
    whole exponent range (a random rotation-like matrix times per-particle
    scales from 2^-60 to 2^60, with per-entry factors from 2^-20 to 2^20,
    zeros, signed zeros and denormals among the entries): the divisions by
    det R and det F run through the shared reciprocal where its safe range
    allows and through the plain division elsewhere, and D must still equal
    the oracle's bit for bit."""
    from material_point_particle_amd import _lib as L
    k = 60_001
    u = G.uniform01(0xE7 + dim, 1, k * dim * dim).reshape(dim * dim, k)
    w = G.uniform01(0xE7 + dim, 2, k * dim * dim).reshape(dim * dim, k)
    z = G.uniform01(0xE7 + dim, 3, k).reshape(1, k)
    scale = np.exp2(np.floor(120.0 * z - 60.0))
    entry = np.exp2(np.floor(40.0 * w - 20.0)) * np.where(u < 0.5, -1.0, 1.0)
    F = (np.eye(dim).reshape(dim * dim, 1) + entry * (u - 0.5)) * scale
    F = F.astype(np.float32)
    F[1, 0:400:3] = 0.0
    F[1, 1:400:3] = -0.0
    F[dim * dim - 1, 400:800] = np.float32(1e-40)      # denormal float32
    D = (np.exp2(np.floor(30.0 * w[::-1] - 25.0)) * (u[::-1] - 0.5)).astype(np.float32)
    D[:, 800:1200] = 0.0
    F, D = np.ascontiguousarray(F), np.ascontiguousarray(D)
    for relax, iters in ((1.5, 12), (1.0, 30)):
        ref = D.copy()
        rst = oracle_lib.pbmpm_project_elastic(dim, F, ref, relax, iters)
        Fd, Dd = dev(F), dev(D)
        st = torch.zeros(4, dtype=torch.int32, device="cuda")
        L.mpm_pbmpm_project_elastic(L.grid_desc(dim, 64, 32), L.particles(k, None, None, Dd, None), Fd, relax,
                                    iters, st)
        torch.cuda.synchronize()
        say("pbmpm projection, wide exponents", dim, relax, iters, rst.tolist())
        assert_same(Dd.cpu().numpy(), ref, f"D ({dim}D, wide exponents, relax {relax}, {iters} Newton steps)")
        assert u32(st).tolist() == rst.tolist()


@pytest.mark.parametrize("restricted", [False, True])
def test_grid_update_bit_exact(mpm, oracle_lib, restricted):
    """The displacement-form update of a P2G grid of the falling jelly cube
    (its bottom near the guardian band after a few substeps' worth of fall)."""
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    w = WORKLOADS["pbmpm_jelly_3d_64"]
    ex = w.extra
    host = build(w)
    host["x"][1] = host["x"][1] - np.float32(1.5 / w.n)        # lower it into the band's reach
    host["v"] = np.ascontiguousarray(host["v"] * np.float32(20.0))
    rng = (w.max_mass, w.max_speed, w.max_affine)
    grid, _ = oracle_lib.p2g_quadratic(3, w.n, w.frac_bits, host, rng)
    dg_ref = oracle_lib.pbmpm_grid_update(3, w.n, grid.copy(), ex["band"])
    parts = DeviceParticles(host)
    tr = Transfer(3, w.n, w.frac_bits, rng, parts.n)
    tr.bin(parts)
    tr.p2g(parts, binned=True)
    from material_point_particle_amd import _lib as L
    L.mpm_pbmpm_grid_update(tr.desc, tr.ws if restricted else None, tr.grid, tr.vg, ex["band"])
    torch.cuda.synchronize()
    say("pbmpm grid update, restricted" if restricted else "pbmpm grid update")
    got = tr.vg.cpu().numpy()
    if restricted:
        m = grid[0] != 0                                    # nodes with mass are all in reached tiles
        assert_same(got[:, m], dg_ref[:, m], "displacement at nodes with mass")
    else:
        assert_same(got, dg_ref, "displacement grid")
    assert int(tr.grid.abs().sum()) == 0
    # the guardian acted on some nodes (displaced positions below 2 dx)
    X = np.arange(w.n, dtype=np.float32) / np.float32(w.n)
    assert np.any(dg_ref[1] + X[None, :, None] == np.float32(2.0 / w.n))


def test_integrate_bit_exact(mpm, oracle_lib):
    from material_point_particle_amd import _lib as L
    k, n = 50_001, 64
    x = (0.02 + 0.96 * G.uniform01(0x1A, 1, 3 * k).reshape(3, k)).astype(np.float32)
    d = (0.02 * (G.uniform01(0x1A, 2, 3 * k).reshape(3, k) - 0.5)).astype(np.float32)
    xr, dr = x.copy(), d.copy()
    rst = oracle_lib.pbmpm_integrate(3, n, xr, dr, 1e-3, (0.0, -9.8, 0.0))
    xd, dd = dev(x), dev(d)
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    L.mpm_pbmpm_integrate(L.grid_desc(3, n, 32), L.particles(k, xd, dd, None, None), 1e-3, (0.0, -9.8, 0.0), st)
    torch.cuda.synchronize()
    assert_same(xd.cpu().numpy(), xr, "x")
    assert_same(dd.cpu().numpy(), dr, "d")
    assert u32(st).tolist() == rst.tolist() and rst[2] > 0


def pbmpm_run(mpm, w, host, substeps):
    from material_point_particle_amd.transfer import ElasticParticles, PBMPMSubsteps, Transfer
    ex = w.extra
    parts = ElasticParticles(host, host["F"], host["vol"])
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    loop = PBMPMSubsteps(tr, parts, ex["dt"], ex["gravity"], ex["iterations"], ex["relax"], ex["polar_iters"],
                         ex["band"])
    return parts, tr, loop


def oracle_state(host):
    return {k: np.ascontiguousarray(host[k].copy()) for k in ("x", "v", "C", "m", "F")}


@pytest.mark.parametrize("form", ["separate", "fused", "records"])
def test_jelly_substeps_in_lockstep(mpm, oracle_lib, form):
    """20 substeps of 5 iterations of the 32,768-particle jelly cube falling
    onto the floor (the guardian engages): after every substep x, d, D and F
    are bit-identical to the oracle's own trajectory, and so is the last
    iteration's P2G grid at every 5th substep.  fused: every iteration's G2P
    but the last runs with the next projection (mpm_pbmpm_g2p_project);
    records: likewise, rewriting the binned records
    (mpm_pbmpm_g2p_project_records), so the substep bins only once, and the
    last G2P with the integrate step and the F update
    (mpm_pbmpm_g2p_integrate)."""
    w = WORKLOADS["pbmpm_jelly_3d_64"]
    ex = w.extra
    host = build(w)
    parts, tr, loop = pbmpm_run(mpm, w, host, ex["substeps"])
    state = oracle_state(host)
    rng = (w.max_mass, w.max_speed, w.max_affine)
    total = np.zeros(4, dtype=np.int64)
    from material_point_particle_amd import _lib as L
    for k in range(1, ex["substeps"] + 1):
        grid_gpu = None
        last = ex["iterations"] - 1
        for it in range(ex["iterations"]):
            # loop.substep(), with the P2G grid of the substep's last iteration kept before the
            # grid update consumes it
            if form == "separate" or it == 0:
                L.mpm_pbmpm_project_elastic(tr.desc, parts.desc(), parts.F, ex["relax"], ex["polar_iters"],
                                            tr.status)
            if form != "records" or it == 0:
                tr.bin(parts)
            tr.p2g(parts, binned=True)
            if it == last and k % 5 == 0:
                grid_gpu = tr.grid.cpu().numpy()
            L.mpm_pbmpm_grid_update(tr.desc, tr.ws, tr.grid, tr.vg, ex["band"])
            if form == "records" and it < last:
                L.mpm_pbmpm_g2p_project_records(tr.desc, tr.vg, parts.desc(), parts.F, ex["relax"],
                                                ex["polar_iters"], tr.ranges, tr.ws, tr.status)
            elif form == "records":
                L.mpm_pbmpm_g2p_integrate(tr.desc, tr.vg, parts.desc(), parts.F, ex["dt"], ex["gravity"], tr.status)
            elif form == "fused" and it < last:
                L.mpm_pbmpm_g2p_project(tr.desc, tr.vg, parts.desc(), parts.F, ex["relax"], ex["polar_iters"],
                                        tr.status)
            else:
                tr.g2p(parts, 0.0)
        if form != "records":
            loop.integrate()
        grid, st = oracle_lib.pbmpm_substep(3, w.n, w.frac_bits, state, rng, ex["iterations"], ex["relax"],
                                            ex["polar_iters"], ex["band"], ex["dt"], ex["gravity"])
        total += st
        torch.cuda.synchronize()
        got = parts.host()
        say("pbmpm lockstep substep", k)
        for key, ref in (("x", state["x"]), ("v", state["v"]), ("C", state["C"]), ("F", state["F"])):
            assert_same(got[key], ref, f"substep {k} {key}")
        if grid_gpu is not None:
            assert_same(grid_gpu, grid, f"substep {k} last iteration's P2G grid")
    # the cube reached the floor: particles pushed back by the guardian, none clamped by the backstop
    assert float(state["x"][1].min()) < 3.0 / w.n
    assert u32(tr.status).tolist()[3] == 0


@pytest.mark.parametrize("dim", [2, 3])
def test_g2p_project_equals_the_two_calls(mpm, dim):
    """mpm_pbmpm_g2p_project against mpm_g2p (dt = 0) followed by
    mpm_pbmpm_project_elastic, on a displacement grid of random values: x, d,
    D and the status counts bit-identical.  Some particles sit outside the
    grid (the gather skips them, the projection still runs on their stored D),
    some at the clamp bounds, some have an inverted F (the projection keeps
    their gathered D)."""
    from material_point_particle_amd import _lib as L
    n, k = (64 if dim == 2 else 32), 50_001
    rng = np.random.default_rng(60 + dim)
    x = rng.uniform(1.0 / n, (n - 2.0) / n, (dim, k)).astype(np.float32)
    x[0, :40] = 0.2 / n                          # base -1 on x: outside the grid
    x[dim - 1, 40:80] = (n - 1.2) / n            # base n - 2 on the last axis: outside
    x[0, 80:120] = 0.9 / n                       # inside the grid, below the clamp bound dx
    d = (0.01 * rng.standard_normal((dim, k))).astype(np.float32)
    D = (0.05 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.1 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    F[0, 120:160] = -3.0                          # det F < 0 for most of these
    dg = (0.002 * rng.standard_normal((dim,) + (n,) * dim)).astype(np.float32)
    desc = L.grid_desc(dim, n, 32)
    out = []
    for fused in (False, True):
        xd, dd, Dd = (torch.from_numpy(a.copy()).cuda() for a in (x, d, D))
        Fd, dgd = torch.from_numpy(F).cuda(), torch.from_numpy(dg).cuda()
        st = torch.zeros(4, dtype=torch.int32, device="cuda")
        parts = L.particles(k, xd, dd, Dd, None)
        if fused:
            L.mpm_pbmpm_g2p_project(desc, dgd, parts, Fd, 1.5, 12, st)
        else:
            L.mpm_g2p(desc, dgd, parts, 0.0, st)
            L.mpm_pbmpm_project_elastic(desc, parts, Fd, 1.5, 12, st)
        torch.cuda.synchronize()
        out.append([a.cpu().numpy() for a in (xd, dd, Dd)] + [u32(st).tolist()])
    say("g2p + projection, one pass", dim, out[1][3])
    for a, b, what in zip(out[0][:3], out[1][:3], ("x", "d", "D")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what
    assert out[0][3] == out[1][3]
    assert out[1][3][0] >= 80 + 20 and out[1][3][2] > 0       # skipped, refused and clamped particles


@pytest.mark.parametrize("dim", [2, 3])
def test_g2p_project_records_rewrites_the_binning(mpm, dim):
    """mpm_pbmpm_g2p_project_records on particles binned beforehand, on a
    displacement grid of random values: x, d, D and the status counts of
    mpm_pbmpm_g2p_project bit for bit; every binned record equal, bit for bit,
    to the record the binning's scatter makes from the new state (x, d, D, m;
    d, D and m zeroed where outside the ranges, which status[1] counts); the
    next P2G on these records bit-identical to a P2G after a fresh binning.
    Particles outside the grid (no record), at the clamp bounds, with an
    inverted F, and outside each of the three ranges before or after the
    gather are included.  A call with other ranges than the binning's is
    refused on the device: status[3] counts it and nothing is written."""
    from material_point_particle_amd import _lib as L
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    n, k = (64 if dim == 2 else 32), 40_003
    rng = np.random.default_rng(70 + dim)
    ranges = (2.0, 0.05, 0.4)
    x = rng.uniform(1.0 / n, (n - 2.0) / n, (dim, k)).astype(np.float32)
    x[0, :40] = 0.2 / n                          # outside the grid
    x[0, 40:80] = 0.9 / n                        # inside, below the clamp bound dx
    x[dim - 1, 80:120] = (n - 1.7) / n           # inside, above the clamp bound (n - 2) dx
    d = (0.01 * rng.standard_normal((dim, k))).astype(np.float32)
    d[0, 120:140] = 0.3                          # d out of range at binning (the gather replaces it)
    D = (0.05 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    D[1, 140:160] = 3.0                          # out of range at binning
    m = rng.uniform(0.5, 1.5, k).astype(np.float32)
    m[160:170] = 5.0                             # out of the mass range for good
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.1 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    F[0, 170:210] = -3.0                         # det F < 0 for most: the gathered D stays
    dg = (0.002 * rng.standard_normal((dim,) + (n,) * dim)).astype(np.float32)
    dg[0, 5:9] = 0.2                             # some gathered d out of range
    host = {"x": x, "v": d, "C": D, "m": m}
    desc = L.grid_desc(dim, n, 32)
    dgd, Fd = dev(dg), dev(F)

    ref = DeviceParticles({kk: a.copy() for kk, a in host.items()})
    st_ref = torch.zeros(4, dtype=torch.int32, device="cuda")
    L.mpm_pbmpm_g2p_project(desc, dgd, ref.desc(), Fd, 1.5, 12, st_ref)

    parts = DeviceParticles({kk: a.copy() for kk, a in host.items()})
    tr = Transfer(dim, n, 32, ranges, k)
    tr.bin(parts)
    torch.cuda.synchronize()
    st_bin = u32(tr.status).copy()
    tr.status.zero_()
    L.mpm_pbmpm_g2p_project_records(desc, dgd, parts.desc(), Fd, 1.5, 12, tr.ranges, tr.ws, tr.status)
    torch.cuda.synchronize()
    st = u32(tr.status).tolist()
    got, want = parts.host(), ref.host()
    for key in ("x", "v", "C"):
        assert np.array_equal(got[key].view(np.uint32), want[key].view(np.uint32)), key
    assert st[0] == u32(st_ref)[0] and st[2] == u32(st_ref)[2] and st[3] == 0
    assert st[0] >= 40 and st[2] > 0

    # the records against the scatter's rule, from the new state
    lay = tr.layout
    R = lay.n_fields
    slot = u32(tr.ws_u32("slot", k)).astype(np.int64)
    has = slot != 0xFFFFFFFF
    assert int(has.sum()) == k - 40 and not has[:40].any()
    recs = tr.ws.view(torch.float32)[lay.sorted // 4: lay.sorted // 4 + R * (int(slot[has].max()) + 1)]
    recs = recs.view(-1, R).cpu().numpy()
    xs, ds, Ds = got["x"], got["v"], got["C"]
    rm, rv, ra = (np.float32(r) for r in ranges)
    inr = (np.abs(m) <= rm) & (np.abs(ds) <= rv).all(0) & (np.abs(Ds) <= ra).all(0)
    exp = np.zeros((k, R), np.float32)
    exp[:, :dim] = xs.T
    exp[:, dim:2 * dim] = ds.T
    exp[:, 2 * dim:2 * dim + dim * dim] = Ds.T
    exp[:, 2 * dim + dim * dim] = m
    exp[~inr, dim:] = 0.0
    assert np.array_equal(recs[slot[has]].view(np.uint32), exp[has].view(np.uint32))
    assert st[1] == int((has & ~inr).sum()) and st[1] > 0
    assert st_bin[1] == int((has & ~((np.abs(m) <= rm) & (np.abs(d) <= rv).all(0)
                                     & (np.abs(D) <= ra).all(0))).sum())
    say("g2p + projection + records", dim, st, "out of range", int((has & ~inr).sum()))

    # the next P2G: refreshed records against a fresh binning of the new state
    g1 = tr.p2g(parts, binned=True).clone()
    tr2 = Transfer(dim, n, 32, ranges, k)
    tr2.bin(parts)
    g2 = tr2.p2g(parts, binned=True)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    assert u32(tr.status)[3] == 0 and u32(tr2.status)[3] == 0

    # other ranges than the binning's: refused on the device, nothing written
    tr.bin(parts)
    torch.cuda.synchronize()
    before = [t.clone() for t in (parts.x, parts.v, parts.C, tr.ws)]
    tr.status.zero_()
    L.mpm_pbmpm_g2p_project_records(desc, dgd, parts.desc(), Fd, 1.5, 12, L.ranges(2.0, 0.06, 0.4), tr.ws,
                                    tr.status)
    torch.cuda.synchronize()
    assert u32(tr.status).tolist() == [0, 0, 0, 1]
    for a, b in zip(before, (parts.x, parts.v, parts.C, tr.ws)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dim", [2, 3])
def test_g2p_integrate_equals_the_three_calls(mpm, dim):
    """mpm_pbmpm_g2p_integrate against mpm_g2p (dt = 0), mpm_pbmpm_integrate
    and mpm_update_deformation (dt = 1) on a displacement grid of random
    values: x, d, D, F and the status counts bit-identical.  Some particles
    sit outside the grid (the gather leaves them; the integrate step and the F
    update still run on them), some below and above the clamp bounds."""
    from material_point_particle_amd import _lib as L
    n, k = (64 if dim == 2 else 32), 50_003
    rng = np.random.default_rng(80 + dim)
    x = rng.uniform(1.0 / n, (n - 2.0) / n, (dim, k)).astype(np.float32)
    x[0, :40] = 0.2 / n
    x[0, 40:80] = 0.9 / n
    x[dim - 1, 80:120] = (n - 1.7) / n
    d = (0.01 * rng.standard_normal((dim, k))).astype(np.float32)
    D = (0.05 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.1 * rng.standard_normal((dim * dim, k))).astype(np.float32)
    dg = (0.02 * rng.standard_normal((dim,) + (n,) * dim)).astype(np.float32)
    grav = (0.0, -9.8, 0.0)[:dim]
    desc = L.grid_desc(dim, n, 32)
    out = []
    for one in (False, True):
        xd, dd, Dd, Fd = (torch.from_numpy(a.copy()).cuda() for a in (x, d, D, F))
        dgd = torch.from_numpy(dg).cuda()
        st = torch.zeros(4, dtype=torch.int32, device="cuda")
        parts = L.particles(k, xd, dd, Dd, None)
        if one:
            L.mpm_pbmpm_g2p_integrate(desc, dgd, parts, Fd, 2e-3, grav, st)
        else:
            L.mpm_g2p(desc, dgd, parts, 0.0, st)
            L.mpm_pbmpm_integrate(desc, parts, 2e-3, grav, st)
            L.mpm_update_deformation(desc, parts, Fd, 1.0)
        torch.cuda.synchronize()
        out.append([a.cpu().numpy() for a in (xd, dd, Dd, Fd)] + [u32(st).tolist()])
    say("g2p + integrate + F update, one launch", dim, out[1][4])
    for a, b, what in zip(out[0][:4], out[1][:4], ("x", "d", "D", "F")):
        assert_same(b, a, what)
    assert out[0][4] == out[1][4]
    assert out[1][4][0] >= 40 and out[1][4][2] > 0


def test_square_2d_substeps_in_lockstep(mpm, oracle_lib):
    """The 2D loop: a 24 x 24-cell elastic square at 4 particles per cell
    (jittered 2 x 2 sub-lattice) thrown down and sideways onto the floor of a
    64^2 grid, 12 substeps of 5 iterations, the guardian engaging; after every
    substep x, d, D and F bit-identical to the oracle's own trajectory."""
    from material_point_particle_amd import _lib as L
    from material_point_particle_amd.transfer import ElasticParticles, PBMPMSubsteps, Transfer
    n, frac, dt, band, iters, relax, polar = 64, 32, 2e-3, 2, 5, 1.5, 12
    cells = np.stack(np.meshgrid(np.arange(20, 44), np.arange(3, 27), indexing="ij"), 0).reshape(2, -1)
    sub = np.stack(np.meshgrid([0.25, 0.75], [0.25, 0.75], indexing="ij"), 0).reshape(2, -1)
    pos = (cells[:, :, None] + sub[:, None, :]).reshape(2, -1)
    k = pos.shape[1]
    jit = 0.2 * (G.uniform01(0x2D, 1, 2 * k).reshape(2, k) - 0.5)
    x = ((pos + jit) / n).astype(np.float32)
    v0 = np.array([0.4, -3.0])[:, None] + 0.05 * (G.uniform01(0x2D, 2, 2 * k).reshape(2, k) - 0.5)
    host = {"x": np.ascontiguousarray(x), "v": np.ascontiguousarray((v0 * dt).astype(np.float32)),
            "C": np.zeros((4, k), np.float32), "m": np.ones(k, np.float32)}
    F = np.ascontiguousarray(np.tile(np.eye(2, dtype=np.float32).reshape(4, 1), (1, k)))
    rng = (1.0, 0.5, 4.0)
    grav = (0.0, -9.8)
    parts = ElasticParticles(host, F, np.full(k, 1.0 / (4 * n * n), np.float32))
    tr = Transfer(2, n, frac, rng, parts.n)
    loop = PBMPMSubsteps(tr, parts, dt, grav, iters, relax, polar, band)
    state = {key: np.ascontiguousarray(a.copy()) for key, a in host.items()}
    state["F"] = F.copy()
    for step in range(1, 13):
        loop.substep()
        oracle_lib.pbmpm_substep(2, n, frac, state, rng, iters, relax, polar, band, dt, grav)
        torch.cuda.synchronize()
        got = parts.host()
        say("pbmpm 2D lockstep substep", step)
        for key in ("x", "v", "C", "F"):
            assert_same(got[key], state[key], f"2D substep {step} {key}")
    assert float(state["x"][1].min()) < 3.0 / n                 # it reached the floor
    assert u32(tr.status).tolist()[0] == 0 and u32(tr.status).tolist()[3] == 0


@pytest.mark.timeout(900)
def test_full_size_jelly_substep(mpm, oracle_lib):
    """One substep (5 iterations) of the 8M-particle jelly cube at 256^3: the
    state and the deformation gradient bit-identical to the oracle's."""
    w = WORKLOADS["pbmpm_jelly_3d_256"]
    ex = w.extra
    host = build(w)
    parts, tr, loop = pbmpm_run(mpm, w, host, 1)
    loop.substep()
    torch.cuda.synchronize()
    got = parts.host()
    say("pbmpm full size: oracle substep")
    state = oracle_state(host)
    oracle_lib.pbmpm_substep(3, w.n, w.frac_bits, state, (w.max_mass, w.max_speed, w.max_affine), ex["iterations"],
                             ex["relax"], ex["polar_iters"], ex["band"], ex["dt"], ex["gravity"])
    for key in ("x", "v", "C", "F"):
        assert_same(got[key], state[key], f"full-size substep {key}")
