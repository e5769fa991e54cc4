"""Pins of the oracle's position-based MPM (PB-MPM) iteration loop for an
elastic material ("Implementation -- GPU Optimization & Reference Codebases",
section 3.3.2): the elastic projection of the displacement gradient D toward
the polar rotation of the trial deformation, the displacement-form grid
update with the guardian, and the integrate step.  Each pin checks the oracle
against mathematics that does not repeat its arithmetic:

- the projection with relaxation 1 lands on a rotation: (I + D') F is
  orthogonal with determinant +1; with a rotation-times-stretch trial whose
  factors are known, it lands on that rotation; a trial that already is a
  rotation is left alone; a symmetric stretch of the rest shape relaxes by the
  factor (1 - relax); the projection commutes with a rotation of the frame;
  inverted trials are refused and counted;
- the grid update's mass normalisation is the exact quotient rounded once, the
  guardian moves exactly the nodes whose displaced position leaves
  [band dx, (n - 1 - band) dx] onto that boundary;
- the integrate step is x + d and d + g dt^2, exact on dyadic values, with
  clamps counted;
- the whole loop: a rigid translation keeps its displacement, a rotated rest
  shape stays put, a consistent linear displacement field is reproduced (with
  relax = 0, the transfer alone), and a stretched free block pulls its faces
  in while its momentum stays zero.
"""
import numpy as np
import pytest

from mpm_inputs import generators as G


def rotation(axis, angle):
    axis = np.asarray(axis, dtype=np.float64)
    axis = axis / np.linalg.norm(axis)
    K = np.array([[0, -axis[2], axis[1]], [axis[2], 0, -axis[0]], [-axis[1], axis[0], 0]])
    return np.eye(3) + np.sin(angle) * K + (1 - np.cos(angle)) * K @ K


def soa(mats):
    """[np][dim][dim] -> float32 component-major [dim*dim][np]."""
    m = np.asarray(mats)
    dim = m.shape[1]
    return np.ascontiguousarray(m.reshape(-1, dim * dim).T.astype(np.float32))


def aos(a, dim):
    return np.asarray(a, dtype=np.float64).T.reshape(-1, dim, dim)


def random_spd(rng, k, dim, spread):
    """k symmetric positive definite matrices with eigenvalues in 1 +- spread."""
    out = []
    for _ in range(k):
        q, _ = np.linalg.qr(rng.normal(size=(dim, dim)))
        lam = 1.0 + spread * (2 * rng.random(dim) - 1)
        out.append(q @ np.diag(lam) @ q.T)
    return np.array(out)


def random_rotations(rng, k, dim):
    out = []
    for _ in range(k):
        q, r = np.linalg.qr(rng.normal(size=(dim, dim)))
        q = q @ np.diag(np.sign(np.diag(r)))
        if np.linalg.det(q) < 0:
            q[:, 0] = -q[:, 0]
        out.append(q)
    return np.array(out)


@pytest.mark.parametrize("dim", [2, 3])
def test_projection_with_relaxation_one_reaches_a_rotation(oracle_lib, dim):
    """relax = 1: D' = R F^-1 - I, so (I + D') F = R, which must be orthogonal
    with det +1 and must be the rotation factor of the trial: R^T Ft is then
    symmetric positive definite (the polar decomposition's stretch)."""
    rng = np.random.default_rng(11 + dim)
    k = 200
    F = random_rotations(rng, k, dim) @ random_spd(rng, k, dim, 0.3)
    D0 = 0.2 * rng.normal(size=(k, dim, dim))
    Ff, Df = soa(F), soa(D0)
    st = oracle_lib.pbmpm_project_elastic(dim, Ff, Df, 1.0, 12)
    assert st.tolist() == [0, 0, 0, 0]
    F64, Dn = aos(Ff, dim), aos(Df, dim)
    Ft = (np.eye(dim) + aos(soa(D0), dim)) @ F64
    R = (np.eye(dim) + Dn) @ F64
    for i in range(k):
        assert np.allclose(R[i].T @ R[i], np.eye(dim), atol=2e-5)
        assert np.linalg.det(R[i]) == pytest.approx(1.0, abs=2e-5)
        S = R[i].T @ Ft[i]
        assert np.allclose(S, S.T, atol=2e-5)
        assert np.all(np.linalg.eigvalsh((S + S.T) / 2) > 0)


def test_projection_recovers_a_known_rotation_and_leaves_rotations_alone(oracle_lib):
    """Trial (I + D) F = Q S with Q a rotation and S symmetric positive
    definite: the target is Q, so with relax = 1, (I + D') F = Q.  A trial that
    is itself a rotation (F = Q, D = 0) needs no change: D' = 0."""
    rng = np.random.default_rng(5)
    k = 50
    Q = np.array([rotation(rng.normal(size=3), rng.uniform(-2.5, 2.5)) for _ in range(k)])
    S = random_spd(rng, k, 3, 0.25)
    F = np.array([np.eye(3) + 0.05 * rng.normal(size=(3, 3)) for _ in range(k)])
    D = Q @ S @ np.linalg.inv(F) - np.eye(3)
    Ff, Df = soa(F), soa(D)
    oracle_lib.pbmpm_project_elastic(3, Ff, Df, 1.0, 12)
    got = (np.eye(3) + aos(Df, 3)) @ aos(Ff, 3)
    assert np.allclose(got, Q, atol=5e-5)
    # a rotation stays a rotation: no change of D (beyond float32 rounding of 0)
    Fq, Dz = soa(Q), soa(np.zeros((k, 3, 3)))
    oracle_lib.pbmpm_project_elastic(3, Fq, Dz, 1.5, 12)
    assert np.abs(Dz).max() < 1e-6


@pytest.mark.parametrize("relax", [0.5, 1.0, 1.5])
def test_symmetric_stretch_of_the_rest_shape_relaxes_by_one_minus_relax(oracle_lib, relax):
    """F = I and a symmetric D with I + D positive definite: the trial is a pure
    stretch, its rotation is I, the target D* = 0, so D' = (1 - relax) D."""
    rng = np.random.default_rng(9)
    k = 100
    D = random_spd(rng, k, 3, 0.2) - np.eye(3)
    F = np.tile(np.eye(3), (k, 1, 1))
    Ff, Df = soa(F), soa(D)
    D32 = aos(Df, 3)
    oracle_lib.pbmpm_project_elastic(3, Ff, Df, relax, 12)
    assert np.allclose(aos(Df, 3), (1 - relax) * D32, atol=2e-6)


def test_projection_commutes_with_a_rotation_of_the_frame(oracle_lib):
    """Rotating the trial deformation by Q0 (D'' with I + D'' = Q0 (I + D))
    rotates the target: R'' = Q0 R, so with relax = 1 the results satisfy
    (I + D1'') F = Q0 (I + D1') F."""
    rng = np.random.default_rng(21)
    k = 60
    F = random_rotations(rng, k, 3) @ random_spd(rng, k, 3, 0.2)
    D = 0.15 * rng.normal(size=(k, 3, 3))
    Q0 = rotation([1.0, 2.0, -0.5], 0.7)
    D2 = Q0 @ (np.eye(3) + D) - np.eye(3)
    Ff = soa(F)
    Da, Db = soa(D), soa(D2)
    oracle_lib.pbmpm_project_elastic(3, Ff, Da, 1.0, 12)
    oracle_lib.pbmpm_project_elastic(3, Ff, Db, 1.0, 12)
    Fa = aos(Ff, 3)
    lhs = (np.eye(3) + aos(Db, 3)) @ Fa
    rhs = Q0 @ (np.eye(3) + aos(Da, 3)) @ Fa
    assert np.allclose(lhs, rhs, atol=5e-5)


def test_inverted_trials_are_refused_and_counted(oracle_lib):
    F = np.tile(np.eye(3), (3, 1, 1))
    D = np.zeros((3, 3, 3))
    D[0] = np.diag([-2.0, 0.0, 0.0])          # (I + D) F has det -1: inverted
    D[1] = np.diag([0.1, -0.2, 0.05])         # fine
    Fb = F.copy()
    Fb[2] = np.diag([-1.0, 1.0, 1.0])         # the stored F itself inverted
    Ff, Df = soa(Fb), soa(D)
    before = Df.copy()
    st = oracle_lib.pbmpm_project_elastic(3, Ff, Df, 1.5, 12)
    assert st.tolist() == [2, 0, 0, 0]
    assert np.array_equal(Df[:, 0], before[:, 0]) and np.array_equal(Df[:, 2], before[:, 2])
    assert not np.array_equal(Df[:, 1], before[:, 1])


def test_grid_update_normalises_and_guards_exactly(oracle_lib):
    """Mass normalisation: d = P/M rounded once to float32.  Guardian: a node
    whose displaced position X + d leaves [band dx, (n - 1 - band) dx] is moved
    onto that bound exactly (d = bound - X); other nodes keep d; massless nodes
    get d = 0; the accumulators are zeroed."""
    n, band = 16, 2
    dx = 1.0 / n
    grid = np.zeros((4, n, n, n), dtype=np.int64)
    M = 3 << 20
    nodes = {(5, 6, 7): (1 << 18, -(1 << 17), 3),           # inside: d = P / M
             (2, 8, 8): (-(M // 2), 0, 0),                   # x = 2 dx at the lower bound, pushed out: clamped
             (13, 8, 8): (M // 4, 0, 0),                     # x = 13 dx = hi: moving out, clamped back
             (12, 8, 8): (M // 32, 0, 0),                    # x = 12 dx, moves 1/32 -> within
             (8, 1, 8): (0, M // 8, 0)}                      # y = 1 dx below lo, moving in by 1/8 = 2 dx: lands on 3 dx
    for (ix, iy, iz), (px, py, pz) in nodes.items():
        grid[0, iz, iy, ix] = M
        grid[1, iz, iy, ix], grid[2, iz, iy, ix], grid[3, iz, iy, ix] = px, py, pz
    dg = oracle_lib.pbmpm_grid_update(3, n, grid, band)
    assert int(np.abs(grid).sum()) == 0
    lo, hi = band * dx, (n - 1 - band) * dx
    for (ix, iy, iz), P in nodes.items():
        for e, (i, p) in enumerate(zip((ix, iy, iz), P)):
            X = i * dx
            d = np.float32(p / M)                                  # exact quotient, rounded once
            want = np.float32(min(max(np.float32(X) + d, np.float32(lo)), np.float32(hi))) - np.float32(X)
            assert dg[e, iz, iy, ix] == want, (ix, iy, iz, e)
    assert dg[0, 8, 8, 2] == np.float32(0.0)                        # pushed out of the lower bound: back to it
    assert dg[0, 8, 8, 13] == np.float32(0.0)                       # at the upper bound, moving out: stays
    assert dg[0, 8, 8, 12] == np.float32(1.0 / 32)
    assert dg[1, 8, 1, 8] == np.float32(2 * dx)                     # 1 dx + 1/8 = 3 dx, inside: kept
    massless = np.ones((n, n, n), dtype=bool)
    for ix, iy, iz in nodes:
        massless[iz, iy, ix] = False
    assert np.all(dg[:, massless] == 0.0)


def test_integrate_moves_by_d_and_adds_gravity(oracle_lib):
    n = 32
    dx = 1.0 / n
    x = np.array([[0.5, 0.5 + dx, 1.5 * dx], [0.25, 0.75, 0.5], [0.5, 0.5, 0.5]], dtype=np.float32)
    d = np.array([[1.0 / 64, -1.0 / 128, -dx], [0.0, 1.0 / 256, 0.0], [-1.0 / 32, 0.0, 0.0]], dtype=np.float32)
    x0, d0 = x.copy(), d.copy()
    dt, g = 0.25, (0.0, -8.0, 2.0)
    st = oracle_lib.pbmpm_integrate(3, n, x, d, dt, g)
    want_x = np.minimum(np.maximum(x0 + d0, np.float32(dx)), np.float32((n - 2) * dx))
    assert np.array_equal(x, want_x)
    assert st.tolist() == [0, 0, 1, 0]                              # the third particle hit x = dx
    gdt2 = np.float32(dt * dt) * np.asarray(g, dtype=np.float32)
    assert np.array_equal(d, d0 + gdt2[:, None])


def cloud(seed, n, count, lo, hi, dim=3):
    """Particles on a jittered lattice (2 per cell per axis) in [lo, hi) cells."""
    cells = int(hi - lo)
    side = 2 * cells
    k = np.arange(side ** dim)
    idx = np.stack([(k // side ** e) % side for e in range(dim)])
    jit = G.uniform01(seed, 1, dim * k.size).reshape(dim, -1)
    x = (lo + (idx + 0.25 + 0.5 * jit) / 2.0) / n
    x = x[:, :count] if count else x
    return np.ascontiguousarray(x.astype(np.float32))


def state_of(x, d, D, F):
    npart = x.shape[1]
    return {"x": x, "v": np.ascontiguousarray(d.astype(np.float32)), "C": np.ascontiguousarray(D.astype(np.float32)),
            "m": np.ones(npart, dtype=np.float32), "F": np.ascontiguousarray(F.astype(np.float32))}


def test_rigid_translation_keeps_its_displacement(oracle_lib):
    """Every particle with the same d, D = 0, F = I, no gravity, far from the
    walls: the transfer reproduces the uniform field (partition of unity), the
    projection has nothing to do, so d stays d0 (to the fixed-point quantum),
    D stays 0 and every particle moves by d0."""
    n = 32
    x = cloud(3, n, 0, 12, 20)
    npart = x.shape[1]
    d0 = np.array([1.0 / 512, -1.0 / 1024, 1.0 / 2048])
    st = state_of(x.copy(), np.tile(d0[:, None], (1, npart)), np.zeros((9, npart)), np.tile(np.eye(3).reshape(9, 1), (1, npart)))
    _, status = oracle_lib.pbmpm_substep(3, n, 32, st, (1.0, 1.0, 1.0), 5, 1.5, 12, 2, 1e-3, (0.0, 0.0, 0.0))
    assert status.tolist() == [0, 0, 0, 0]
    assert np.abs(st["v"] - d0[:, None]).max() < 1e-8
    assert np.abs(st["C"]).max() < 1e-5
    assert np.abs(st["x"] - (x + d0[:, None].astype(np.float32))).max() < 1e-7


def test_rotated_rest_shape_stays_put(oracle_lib):
    """F = Q (a rotation), d = 0, D = 0: nothing is strained, so nothing moves
    and F stays Q."""
    n = 32
    x = cloud(4, n, 0, 12, 20)
    npart = x.shape[1]
    Q = rotation([0.3, -1.0, 0.5], 0.9)
    st = state_of(x.copy(), np.zeros((3, npart)), np.zeros((9, npart)), np.tile(Q.reshape(9, 1), (1, npart)))
    oracle_lib.pbmpm_substep(3, n, 32, st, (1.0, 1.0, 1.0), 5, 1.5, 12, 2, 1e-3, (0.0, 0.0, 0.0))
    assert np.abs(st["v"]).max() < 1e-9 and np.abs(st["C"]).max() < 1e-6
    assert np.array_equal(st["x"], x)
    assert np.allclose(aos(st["F"], 3), Q, atol=1e-6)


def test_consistent_linear_field_is_reproduced_by_the_loop(oracle_lib):
    """With relax = 0 the projection leaves D alone and the loop is the
    transfer repeated: a consistent linear displacement field, d_p = A x_p + b
    and D_p = A with A not symmetric, is reproduced by P2G, the grid update and
    the G2P gather at every iteration (linear reproduction of the quadratic
    B-spline: sum w x_i = x_p, sum w (x_i - x_p)(x_i - x_p)^T = dx^2/4 I), to
    float32 rounding; then x += d and F <- (I + A) F.  (The gathered D carries
    ~1e-6 relative float32 error: B = sum w vg r cancels to ~1/400 of its
    terms; through d + D r it moves d by ~1e-8 per iteration.)"""
    n = 32
    x = cloud(6, n, 0, 10, 22)
    npart = x.shape[1]
    A = np.array([[2e-3, -1e-3, 5e-4], [1.5e-3, -1e-3, 0.0], [-5e-4, 2.5e-3, 1e-3]])
    b = np.array([1e-4, -2e-4, 3e-4])
    d = (A @ x.astype(np.float64) + b[:, None]).astype(np.float32)
    st = state_of(x.copy(), d, np.tile(A.reshape(9, 1), (1, npart)), np.tile(np.eye(3).reshape(9, 1), (1, npart)))
    d32 = st["v"].astype(np.float64)
    _, status = oracle_lib.pbmpm_substep(3, n, 32, st, (1.0, 1.0, 1.0), 3, 0.0, 12, 2, 1e-3, (0.0, 0.0, 0.0))
    assert status.tolist() == [0, 0, 0, 0]
    assert np.abs(st["v"] - d32).max() < 5e-8
    assert np.abs(aos(st["C"], 3) - A).max() < 2e-6
    assert np.abs(st["x"] - (x + d32.astype(np.float32))).max() < 2e-7
    assert np.allclose(aos(st["F"], 3), np.eye(3) + A, atol=2e-6)


@pytest.mark.parametrize("relax", [1.0, 1.5])
def test_stretched_free_block_pulls_its_faces_in_and_keeps_its_momentum(oracle_lib, relax):
    """A free block stored with F = s I (s = 1.1, stretched), d = D = 0, no
    gravity, far from the walls.  The projection asks every particle for
    D* = I/s - I (a contraction); the grid couples the particles, so after a
    substep the block's faces have moved inward, the block is mirror-symmetric
    about its centre (its particles are), and the total momentum sum m d stays
    zero (the transfer conserves it: sum_i w_i (x_i - x_p) = 0), to the
    fixed-point quantum."""
    n = 64
    s = 1.1
    x = cloud(5, n, 0, 24, 40)
    xs = x * n
    # a mirror-symmetric block: each particle and its reflection about the centre
    centre = 32.0
    x = np.ascontiguousarray(np.concatenate([x, (2 * centre - xs) / n], axis=1).astype(np.float32))
    npart = x.shape[1]
    st = state_of(x.copy(), np.zeros((3, npart)), np.zeros((9, npart)), np.tile((s * np.eye(3)).reshape(9, 1), (1, npart)))
    oracle_lib.pbmpm_substep(3, n, 32, st, (1.0, 1.0, 1.0), 5, relax, 12, 2, 1e-3, (0.0, 0.0, 0.0))
    dx_ = st["x"].astype(np.float64) - x.astype(np.float64)
    assert np.abs(dx_.sum(axis=1)).max() < 1e-9 * npart       # momentum (unit masses): zero to the quantum
    xs = x.astype(np.float64) * n
    for e in range(3):
        hi_face = xs[e] > 39.0
        lo_face = xs[e] < 25.0
        assert np.all(dx_[e, hi_face] < 0) and np.all(dx_[e, lo_face] > 0)
    extent_before = xs.max(axis=1) - xs.min(axis=1)
    after = st["x"].astype(np.float64) * n
    assert np.all(after.max(axis=1) - after.min(axis=1) < extent_before)
