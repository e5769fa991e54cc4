"""Pins for the oracle's MLS-MPM stress term (Neo-Hookean solid) and the
deformation-gradient update.

"Implementation -- GPU Optimization & Reference Codebases", section 3.1, part 2
of the guide described there: with J = det F and F^-T = (F^T)^-1,
P = mu (F - F^-T) + lambda log(J) F^-T and sigma = (1/J) P F^T.  The stress
enters P2G through the affine matrix, C' = C - k (P F^T) with
k = dt vol0 4 n^2 / m, and F is advanced after G2P as F <- (I + dt C) F.

The pins are independent of the oracle's arithmetic: closed forms for uniform
dilation and simple shear, the energy the stress derives from (finite
differences of the Neo-Hookean energy density in float64), frame
indifference, symmetry of the Kirchhoff stress, exact dyadic cases of the F
update and det(F') = det(I + dt C) det(F), and momentum conservation of a P2G
that carries the stress term.
"""
import numpy as np
import pytest

from mpm_inputs import generators as G

N = 64
DT, MU, LAM = 1e-4, 3.0e5, 5.0e5


def tau_of(oracle_lib, dim, F, vol0=1e-6, m=1.0):
    """Kirchhoff stress P F^T recovered from C' with C = 0: tau = -C' / k."""
    np_ = F.shape[-1]
    parts = {"x": np.zeros((dim, np_), np.float32), "v": np.zeros((dim, np_), np.float32),
             "C": np.zeros((dim * dim, np_), np.float32), "m": np.full(np_, m, np.float32)}
    out, st = oracle_lib.neohookean_affine(dim, N, parts, F.reshape(dim * dim, np_), np.full(np_, vol0, np.float32),
                                           DT, MU, LAM)
    k = (DT * np.float64(np.float32(vol0)) * 4.0 * N * N) / m
    return -out.astype(np.float64).reshape(dim, dim, np_) / k, st


def energy(F, dim, mu=MU, lam=LAM):
    """Neo-Hookean energy density: mu/2 (tr F^T F - dim) - mu log J + lam/2 (log J)^2."""
    J = np.linalg.det(F)
    return 0.5 * mu * (np.trace(F.T @ F) - dim) - mu * np.log(J) + 0.5 * lam * np.log(J) ** 2


@pytest.mark.parametrize("dim", [2, 3])
def test_identity_deformation_leaves_C(oracle_lib, dim):
    np_ = 50
    C = G.normal(11, 1, dim * dim * np_, 1.0).reshape(dim * dim, np_).astype(np.float32)
    F = np.tile(np.eye(dim, dtype=np.float32).reshape(dim * dim, 1), (1, np_))
    parts = {"x": np.zeros((dim, np_), np.float32), "v": np.zeros((dim, np_), np.float32), "C": C,
             "m": np.ones(np_, np.float32)}
    out, st = oracle_lib.neohookean_affine(dim, N, parts, F, np.full(np_, 1e-6, np.float32), DT, MU, LAM)
    assert np.array_equal(out, C) and st.tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("dim", [2, 3])
def test_uniform_dilation_closed_form(oracle_lib, dim):
    """F = s I: tau = (mu (s^2 - 1) + dim lambda log s) I."""
    s = np.array([0.8, 0.95, 1.0, 1.05, 1.3], np.float32)
    F = np.zeros((dim, dim, s.size), np.float32)
    for d in range(dim):
        F[d, d] = s
    tau, st = tau_of(oracle_lib, dim, F)
    s64 = s.astype(np.float64)
    want = MU * (s64 ** 2 - 1) + dim * LAM * np.log(s64)
    for d in range(dim):
        for e in range(dim):
            if d == e:
                assert np.allclose(tau[d, e], want, rtol=1e-6, atol=1e-3)
            else:
                assert np.all(tau[d, e] == 0)
    assert st.tolist() == [0, 0, 0, 0]


def test_simple_shear_closed_form(oracle_lib):
    """F = I + g e_x e_y^T: J = 1, tau = mu [[g^2, g, 0], [g, 0, 0], [0, 0, 0]]."""
    g = np.array([0.1, -0.25, 0.5], np.float32)
    F = np.zeros((3, 3, g.size), np.float32)
    for d in range(3):
        F[d, d] = 1
    F[0, 1] = g
    tau, _ = tau_of(oracle_lib, 3, F)
    g64 = g.astype(np.float64)
    want = np.zeros((3, 3, g.size))
    want[0, 0], want[0, 1], want[1, 0] = MU * g64 ** 2, MU * g64, MU * g64
    assert np.allclose(tau, want, rtol=1e-6, atol=1e-3)


@pytest.mark.parametrize("dim", [2, 3])
def test_stress_is_the_energy_derivative(oracle_lib, dim):
    """P = dPsi/dF by central differences of the energy (float64), and
    tau = P F^T recovered from C'."""
    rng = np.random.default_rng(7)
    Fs = np.eye(dim)[:, :, None] + 0.15 * rng.standard_normal((dim, dim, 20))
    Fs = Fs.astype(np.float32)
    tau, st = tau_of(oracle_lib, dim, Fs)
    for p in range(Fs.shape[-1]):
        F = Fs[:, :, p].astype(np.float64)
        if np.linalg.det(F) <= 0:
            continue
        P = np.zeros((dim, dim))
        h = 1e-6
        for d in range(dim):
            for e in range(dim):
                Fp, Fm = F.copy(), F.copy()
                Fp[d, e] += h
                Fm[d, e] -= h
                P[d, e] = (energy(Fp, dim) - energy(Fm, dim)) / (2 * h)
        assert np.allclose(tau[:, :, p], P @ F.T, rtol=1e-5, atol=1e-2 * MU * 1e-3)


def test_frame_indifference_and_symmetry(oracle_lib):
    """tau(Q F) = Q tau(F) Q^T for a rotation Q, and tau = tau^T."""
    rng = np.random.default_rng(3)
    F = (np.eye(3)[:, :, None] + 0.2 * rng.standard_normal((3, 3, 16)))
    th = 0.7
    Q = np.array([[np.cos(th), -np.sin(th), 0], [np.sin(th), np.cos(th), 0], [0, 0, 1]])
    QF = np.einsum("de,eqp->dqp", Q, F)
    t1, _ = tau_of(oracle_lib, 3, F.astype(np.float32))
    t2, _ = tau_of(oracle_lib, 3, QF.astype(np.float32))
    scale = np.abs(t1).max()
    for p in range(F.shape[-1]):
        if np.linalg.det(F[:, :, p]) <= 0:
            continue
        assert np.allclose(t2[:, :, p], Q @ t1[:, :, p] @ Q.T, rtol=1e-4, atol=1e-5 * scale)
        assert np.allclose(t1[:, :, p], t1[:, :, p].T, rtol=1e-6, atol=1e-7 * scale)


@pytest.mark.parametrize("dim", [2, 3])
def test_inverted_and_massless_particles_keep_C(oracle_lib, dim):
    np_ = 4
    F = np.tile(np.eye(dim, dtype=np.float32).reshape(dim * dim, 1), (1, np_))
    F[0, 0] = -1.0                      # particle 0 inverted (det < 0)
    F[0, 1] = 0.0                       # particle 1 degenerate (det = 0)
    F[0, 2] = 1.2                       # particle 2 stretched, massless
    F[0, 3] = 1.2                       # particle 3 stretched, with mass
    C = np.full((dim * dim, np_), 0.25, np.float32)
    parts = {"x": np.zeros((dim, np_), np.float32), "v": np.zeros((dim, np_), np.float32), "C": C,
             "m": np.array([1, 1, 0, 1], np.float32)}
    out, st = oracle_lib.neohookean_affine(dim, N, parts, F, np.full(np_, 1e-6, np.float32), DT, MU, LAM)
    assert np.array_equal(out[:, :3], C[:, :3])
    assert not np.array_equal(out[:, 3], C[:, 3])
    assert st.tolist() == [2, 0, 0, 0]


@pytest.mark.parametrize("dim", [2, 3])
def test_update_F_exact_and_determinant(oracle_lib, dim):
    """Dyadic C and dt: F' = (I + dt C) F is exact; in general
    det F' = det(I + dt C) det F to rounding."""
    rng = np.random.default_rng(5)
    np_ = 30
    C = (rng.integers(-8, 9, (dim * dim, np_)) / 8.0).astype(np.float32)
    F = (rng.integers(-8, 9, (dim * dim, np_)) / 8.0).astype(np.float32)
    for d in range(dim):
        F[d * dim + d] += 2.0
    F0 = F.copy()
    oracle_lib.update_F(dim, C, F, 1.0 / 16)
    for p in range(np_):
        Gm = np.eye(dim) + C[:, p].reshape(dim, dim).astype(np.float64) / 16
        want = Gm @ F0[:, p].reshape(dim, dim).astype(np.float64)
        assert np.array_equal(F[:, p].reshape(dim, dim).astype(np.float64), want)
    C2 = rng.standard_normal((dim * dim, np_)).astype(np.float32)
    F2 = (np.eye(dim).reshape(dim * dim, 1) + 0.3 * rng.standard_normal((dim * dim, np_))).astype(np.float32)
    F20 = F2.copy()
    oracle_lib.update_F(dim, C2, F2, 1e-3)
    for p in range(np_):
        Gm = np.eye(dim) + 1e-3 * C2[:, p].reshape(dim, dim).astype(np.float64)
        d0 = np.linalg.det(F20[:, p].reshape(dim, dim).astype(np.float64))
        d1 = np.linalg.det(F2[:, p].reshape(dim, dim).astype(np.float64))
        assert abs(d1 - np.linalg.det(Gm) * d0) <= 1e-5 * max(1.0, abs(d0))


def test_p2g_with_stress_conserves_momentum(oracle_lib):
    """The stress term's node contributions sum to zero (sum_i w_i (x_i - x_p)
    = 0), so the grid's total momentum is sum m v within the rounding bound."""
    dim, n, k, np_ = 3, 32, 24, 2000
    rng = np.random.default_rng(9)
    x = rng.uniform(0.2, 0.8, (dim, np_)).astype(np.float32)
    v = rng.standard_normal((dim, np_)).astype(np.float32)
    C = (0.1 * rng.standard_normal((dim * dim, np_))).astype(np.float32)
    m = rng.uniform(0.5, 2.0, np_).astype(np.float32)
    F = (np.eye(dim).reshape(dim * dim, 1) + 0.1 * rng.standard_normal((dim * dim, np_))).astype(np.float32)
    parts = {"x": x, "v": v, "C": C, "m": m}
    Cs, st = oracle_lib.neohookean_affine(dim, n, parts, F, np.full(np_, 1.0 / n ** 3, np.float32), 1e-3, 1e4,
                                          1e4)
    assert st[0] == 0 and np.abs(Cs - C).max() > 1.0              # the stress term is not negligible here
    grid, status = oracle_lib.p2g_quadratic(dim, n, k, {"x": x, "v": v, "C": Cs, "m": m}, (1e3, 1e3, 1e6))
    assert status.tolist() == [0, 0, 0, 0]
    S = 2.0 ** k
    want = (m.astype(np.float64)[None] * v.astype(np.float64)).sum(axis=1) * S
    got = grid[1:].reshape(dim, -1).sum(axis=1).astype(np.float64)
    # per contribution: rounding to the quantum (1/2) plus float32 products (relative 2^-22 of its size)
    bound = np_ * 27 * (0.5 + 2.0 ** -21 * S * 2.0 * (1 + np.abs(Cs).max()))
    assert np.all(np.abs(got - want) <= bound), (got - want, bound)
