"""GPU parity of the MLS-MPM stress term (Neo-Hookean solid) and the
deformation-gradient update against the oracle, through the C ABI.

The stress is formed in float64 with the same operation order on both sides;
the only operation whose last bit may differ between the host's and the
device's math library is the float64 log, so C' may differ from the oracle by
at most one float32 ulp, in a vanishing fraction of entries.  Everything else
(the F update, and P2G, grid update and G2P given the same C') is bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

from mpm_inputs import WORKLOADS, build

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


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def assert_close_ulp(gpu, ref, what, max_frac=1e-4):
    d = ulp_diff(gpu, ref)
    assert d.max() <= 1, f"{what}: {d.max()} ulp apart"
    assert np.count_nonzero(d) <= max(1, int(max_frac * d.size)), f"{what}: {np.count_nonzero(d)} entries 1 ulp apart"


def random_solid(dim, np_, seed, inverted=0):
    rng = np.random.default_rng(seed)
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.2 * rng.standard_normal((dim * dim, np_))).astype(np.float32)
    if inverted:
        F[0, :inverted] = -np.abs(F[0, :inverted]) - 2.0      # det < 0 for the first few (dominant -F00)
        for q in range(1, dim):
            F[q * dim + q, :inverted] = 1.0
            F[q, :inverted] = 0.0
            F[q * dim, :inverted] = 0.0
    host = {"x": rng.uniform(0.2, 0.8, (dim, np_)).astype(np.float32),
            "v": rng.standard_normal((dim, np_)).astype(np.float32),
            "C": rng.standard_normal((dim * dim, np_)).astype(np.float32),
            "m": rng.uniform(0.5, 2.0, np_).astype(np.float32)}
    host["m"][-3:] = 0.0
    vol0 = rng.uniform(0.5, 2.0, np_).astype(np.float32) * 1e-6
    return host, F, vol0


@pytest.mark.parametrize("dim", [2, 3])
def test_neohookean_affine_matches_oracle(mpm, oracle_lib, dim):
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    np_ = 100_003
    host, F, vol0 = random_solid(dim, np_, 21 + dim, inverted=17)
    dt, mu, lam = 1e-4, 2.0e8, 3.0e8
    n = 64
    say("neohookean affine", dim, np_)
    ref, ref_st = oracle_lib.neohookean_affine(dim, n, host, F, vol0, dt, mu, lam)
    parts = ElasticParticles(host, F, vol0)
    tr = Transfer(dim, n, 24, (2.0, 10.0, 1e6), np_)
    parts.stress(tr, dt, mu, lam)
    torch.cuda.synchronize()
    got = parts.C_aff.cpu().numpy()
    assert_close_ulp(got, ref, "C'")
    assert tr.status.cpu().numpy().view(np.uint32).tolist() == ref_st.tolist()
    assert ref_st[0] >= 17                      # the 17 built inverted, and any the random draw inverted
    # inverted and massless particles keep C exactly
    assert np.array_equal(got[:, :17], host["C"][:, :17]) and np.array_equal(got[:, -3:], host["C"][:, -3:])


@pytest.mark.parametrize("dim", [2, 3])
def test_update_F_bit_exact(mpm, oracle_lib, dim):
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    np_ = 65_537
    host, F, vol0 = random_solid(dim, np_, 31 + dim)
    ref = F.copy()
    oracle_lib.update_F(dim, host["C"], ref, 1e-3)
    parts = ElasticParticles(host, F, vol0)
    tr = Transfer(dim, 32, 24, (2.0, 10.0, 10.0), np_)
    say("update F", dim)
    parts.update_F(tr, 1e-3)
    torch.cuda.synchronize()
    assert np.array_equal(parts.F.cpu().numpy(), ref)


@pytest.mark.parametrize("dim", [2, 3])
def test_fused_update_and_stress_equals_the_two_calls(mpm, oracle_lib, dim):
    """mpm_update_deformation_stress against mpm_update_deformation followed
    by mpm_neohookean_affine on the same inputs: F and C' bit-identical, the
    same status count; against the oracle, F bit-exact and C' within one
    float32 ulp (float64 log).  Some particles are inverted after the update
    (det F <= 0 keeps C), some massless."""
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    np_ = 70_001
    host, F, vol0 = random_solid(dim, np_, 41 + dim, inverted=23)
    host["C"] *= 30.0                            # large enough that dt C moves F visibly
    dt, mu, lam = 2e-3, 2.0e8, 3.0e8
    n = 64
    say("fused F update and stress", dim, np_)
    sep = ElasticParticles(host, F, vol0)
    fus = ElasticParticles(host, F, vol0)
    tr_s = Transfer(dim, n, 24, (2.0, 10.0, 1e6), np_)
    tr_f = Transfer(dim, n, 24, (2.0, 10.0, 1e6), np_)
    sep.update_F(tr_s, dt)
    sep.stress(tr_s, dt, mu, lam)
    fus.update_F_stress(tr_f, dt, mu, lam)
    torch.cuda.synchronize()
    F_sep, F_fus = sep.F.cpu().numpy(), fus.F.cpu().numpy()
    c_sep, c_fus = sep.C_aff.cpu().numpy(), fus.C_aff.cpu().numpy()
    assert np.array_equal(F_fus.view(np.uint32), F_sep.view(np.uint32))
    assert np.array_equal(c_fus.view(np.uint32), c_sep.view(np.uint32))
    st = tr_f.status.cpu().numpy().view(np.uint32).tolist()
    assert st == tr_s.status.cpu().numpy().view(np.uint32).tolist() and st[0] >= 23
    F_ref = F.copy()
    oracle_lib.update_F(dim, host["C"], F_ref, dt)
    assert np.array_equal(F_fus, F_ref)
    ref, ref_st = oracle_lib.neohookean_affine(dim, n, host, F_ref, vol0, dt, mu, lam)
    assert_close_ulp(c_fus, ref, "C'")
    assert ref_st.tolist() == st


@pytest.mark.parametrize("dim", [2, 3])
def test_g2p_update_stress_equals_the_two_calls(mpm, dim):
    """mpm_g2p_update_deformation_stress against mpm_g2p followed by
    mpm_update_deformation_stress on the same inputs and a grid velocity of
    random values: x, v, C, F and C' bit-identical, the same status counts.
    Some particles sit outside the grid (the gather leaves them, the F update
    still runs on their C), some at the clamp bounds, some are inverted after
    the update, some massless."""
    from material_point_particle_amd import _lib as L
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    np_, n = 60_001, (64 if dim == 2 else 32)
    host, F, vol0 = random_solid(dim, np_, 77 + dim, inverted=31)
    rng = np.random.default_rng(90 + dim)
    host["x"] = rng.uniform(1.0 / n, (n - 2.0) / n, (dim, np_)).astype(np.float32)
    host["x"][0, 31:70] = 0.2 / n                           # outside the grid
    host["x"][dim - 1, 70:110] = (n - 1.7) / n              # inside, above the clamp bound
    host["C"] *= 30.0
    vg = (0.5 * rng.standard_normal((dim,) + (n,) * dim)).astype(np.float32)
    dt, mu, lam = 2e-3, 2.0e8, 3.0e8
    out = []
    for one in (False, True):
        parts = ElasticParticles(host, F, vol0)
        tr = Transfer(dim, n, 24, (2.0, 10.0, 1e6), np_)
        tr.vg.copy_(torch.from_numpy(vg))
        if one:
            parts.g2p_update_F_stress(tr, dt, mu, lam)
        else:
            tr.g2p(parts, dt)
            parts.update_F_stress(tr, dt, mu, lam)
        torch.cuda.synchronize()
        out.append([t.cpu().numpy().view(np.uint32) for t in (parts.x, parts.v, parts.C, parts.F, parts.C_aff)]
                   + [tr.status.cpu().numpy().view(np.uint32).tolist()])
    say("G2P with the F update and stress, one launch", dim, out[1][5])
    for a, b, what in zip(out[0][:5], out[1][:5], ("x", "v", "C", "F", "C'")):
        assert np.array_equal(a, b), what
    assert out[0][5] == out[1][5]
    st = out[1][5]
    assert st[0] >= 39 + 31 and st[2] > 0                  # outside, inverted; clamped


@pytest.mark.parametrize("form", ["separate", "fused", "one_launch"])
def test_elastic_substeps_match_oracle(mpm, oracle_lib, form):
    """An elastic cube thrown at the floor (32,768 particles, 64^3 nodes): the
    substep stress -> bin -> P2G (with C') -> restricted grid update -> G2P ->
    F update on the GPU (fused: the F update and the next substep's stress in
    one call after G2P, the first substep's stress on its own; one_launch: G2P
    and that call as one, mpm_g2p_update_deformation_stress).  At every 10th
    substep the oracle recomputes that substep from the GPU's state before it:
    C' within one ulp (float64 log); given the GPU's C', the P2G grid, the
    particle state and F bit-exact."""
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    w = WORKLOADS["jelly_3d_64"]
    ex = w.extra
    host = build(w)
    parts = ElasticParticles(host, host["F"], host["vol"])
    rng = (w.max_mass, w.max_speed, w.max_affine)
    tr = Transfer(w.dim, w.n, w.frac_bits, rng, parts.n)
    checked = 0
    for k in range(1, ex["substeps"] + 1):
        check = k % ex["check_every"] == 0
        if check:
            torch.cuda.synchronize()
            before = parts.host()
        if form == "separate" or k == 1:
            parts.stress(tr, ex["dt"], ex["mu"], ex["lam"])
        tr.bin(parts.affine())
        tr.p2g(parts.affine(), binned=True)
        if check:
            torch.cuda.synchronize()
            c_aff = parts.C_aff.cpu().numpy()
            grid = tr.grid.cpu().numpy()
        tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
        if form == "one_launch":
            parts.g2p_update_F_stress(tr, ex["dt"], ex["mu"], ex["lam"])
        else:
            tr.g2p(parts, ex["dt"])
            if form == "fused":
                parts.update_F_stress(tr, ex["dt"], ex["mu"], ex["lam"])
            else:
                parts.update_F(tr, ex["dt"])
        if not check:
            continue
        torch.cuda.synchronize()
        after = parts.host()
        say("elastic substep", k, form)
        ref_c, _ = oracle_lib.neohookean_affine(3, w.n, before, before["F"], host["vol"], ex["dt"], ex["mu"],
                                                ex["lam"])
        assert_close_ulp(c_aff, ref_c, f"C' at substep {k}")
        st = {"x": before["x"].copy(), "v": before["v"].copy(), "C": c_aff.copy(), "m": before["m"].copy()}
        g_ref, s_ref = oracle_lib.p2g_quadratic(3, w.n, w.frac_bits, st, rng)
        assert np.array_equal(grid, g_ref), f"P2G grid at substep {k}"
        assert s_ref.tolist() == [0, 0, 0, 0]
        vg = oracle_lib.grid_update(3, w.n, g_ref, ex["dt"], ex["gravity"], ex["sticky"])
        st["C"] = before["C"].copy()
        oracle_lib.g2p(3, w.n, vg, st, ex["dt"])
        F_ref = before["F"].copy()
        oracle_lib.update_F(3, st["C"], F_ref, ex["dt"])
        for key in ("x", "v", "C"):
            assert np.array_equal(after[key], st[key]), f"{key} at substep {k}"
        assert np.array_equal(after["F"], F_ref), f"F at substep {k}"
        checked += 1
    assert checked == ex["substeps"] // ex["check_every"]
    # the cube has hit the floor and is deforming: some particles are compressed
    J = np.linalg.det(parts.F.cpu().numpy().reshape(3, 3, -1).transpose(2, 0, 1))
    assert J.min() < 0.999 and np.all(J > 0)


@pytest.mark.timeout(900)
def test_elastic_full_size_checked_substeps(mpm, oracle_lib):
    """The benchmark's elastic workload at full size (8M-particle jelly cube,
    256^3 nodes) in the benchmark's loop (G2P, the F update and the next
    substep's stress in one launch): 12 substeps on the GPU; substeps 6 and 12 are
    recomputed by the oracle from the GPU state before them: C' within one
    float32 ulp, and given the GPU's C', the P2G grid, the particles and F
    bit-exact."""
    from material_point_particle_amd.transfer import ElasticParticles, Transfer
    w = WORKLOADS["jelly_3d_256"]
    ex = w.extra
    host = build(w)
    vol = host["vol"]
    parts = ElasticParticles(host, host["F"], vol)
    del host
    rng = (w.max_mass, w.max_speed, w.max_affine)
    tr = Transfer(w.dim, w.n, w.frac_bits, rng, parts.n)
    for k in range(1, 13):
        check = k in (6, 12)
        if check:
            torch.cuda.synchronize()
            before = parts.host()
        if k == 1:
            parts.stress(tr, ex["dt"], ex["mu"], ex["lam"])
        tr.bin(parts.affine())
        tr.p2g(parts.affine(), binned=True)
        if check:
            torch.cuda.synchronize()
            c_aff = parts.C_aff.cpu().numpy()
            grid = tr.grid.cpu().numpy()
        tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
        parts.g2p_update_F_stress(tr, ex["dt"], ex["mu"], ex["lam"])
        if not check:
            continue
        torch.cuda.synchronize()
        after = parts.host()
        say("elastic full size, substep", k)
        ref_c, _ = oracle_lib.neohookean_affine(3, w.n, before, before["F"], vol, ex["dt"], ex["mu"], ex["lam"])
        assert_close_ulp(c_aff, ref_c, f"C' at substep {k}")
        del ref_c
        st = {"x": before["x"], "v": before["v"], "C": c_aff, "m": before["m"]}
        g_ref, s_ref = oracle_lib.p2g_quadratic(3, w.n, w.frac_bits, st, rng)
        assert np.array_equal(grid, g_ref), f"P2G grid at substep {k}"
        assert s_ref.tolist() == [0, 0, 0, 0]
        del grid
        vg = oracle_lib.grid_update(3, w.n, g_ref, ex["dt"], ex["gravity"], ex["sticky"])
        del g_ref
        st = {"x": before["x"].copy(), "v": before["v"].copy(), "C": before["C"].copy(), "m": before["m"]}
        oracle_lib.g2p(3, w.n, vg, st, ex["dt"])
        F_ref = before["F"].copy()
        oracle_lib.update_F(3, st["C"], F_ref, ex["dt"])
        for key in ("x", "v", "C"):
            assert np.array_equal(after[key], st[key]), f"{key} at substep {k}"
        assert np.array_equal(after["F"], F_ref), f"F at substep {k}"
