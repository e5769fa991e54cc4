"""The five seeded P2G workloads, each a plain description plus a builder.

A workload fixes the grid (dimension, nodes per axis, fixed-point scale,
tile edge), the particle count, the declared value ranges that the bounds
check needs, and how particles are placed and given mass, velocity and an
affine matrix.  Arrays use the component-major layout both implementations
read: ``x[d][N]``, ``v[d][N]``, ``C[d*dim+e][N]`` (row d, column e of the
affine matrix), ``m[N]``, all float32 and C-contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

from . import generators as G


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "cic_split", "quadratic" or "isplit"
    dim: int
    n: int                    # nodes per axis (quadratic); cells per axis (cic_split)
    n_particles: int
    frac_bits: int            # fixed-point scale S = 2**frac_bits
    tile: int = 4             # tile edge in cells for binning
    placement: str = ""
    mass: object = 1.0        # constant, or (lo, hi) uniform
    v_sigma: float = 0.0
    c_sigma: float = 0.0
    max_mass: float = 0.0     # declared ranges: |m| <= max_mass, |v_d| <= max_speed,
    max_speed: float = 0.0    # |C_de| <= max_affine (particles outside are skipped
    max_affine: float = 0.0   # and counted)
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def channels(self) -> int:
        return 1 + self.dim

    @property
    def nodes(self) -> int:
        if self.kind == "cic_split":
            return (self.n + 1) ** 2
        return self.n ** self.dim


def _seed(i: int) -> int:
    return 0x4D504D00 + i


WORKLOADS = {
    # 2D integer-split cloud-in-cell: 256 particles on 8x8 cells (9x9 nodes).
    "cic_split_2d": Workload(
        name="cic_split_2d", kind="cic_split", dim=2, n=8, n_particles=256, frac_bits=16,
        max_mass=1000, max_speed=1000, seed=_seed(1)),
    # 2D APIC, quadratic stencil: a 3,500-particle settled pile on 64x64 nodes.
    "pile_2d": Workload(
        name="pile_2d", kind="quadratic", dim=2, n=64, n_particles=3500, frac_bits=32,
        placement="pile", mass=1.0, v_sigma=0.5, c_sigma=0.1,
        max_mass=1.0, max_speed=4.0, max_affine=1.0, seed=_seed(2)),
    # 3D dam-break block, 1M particles, 128^3 nodes.
    "dam_3d_128": Workload(
        name="dam_3d_128", kind="quadratic", dim=3, n=128, n_particles=1 << 20, frac_bits=32,
        placement="dam", mass=1.0, v_sigma=0.1, c_sigma=0.05,
        max_mass=1.0, max_speed=1.0, max_affine=0.5, seed=_seed(3)),
    # 3D contention stress: 16M particles in 32 Gaussian blobs, 256^3 nodes.
    "blobs_3d_256": Workload(
        name="blobs_3d_256", kind="quadratic", dim=3, n=256, n_particles=1 << 24, frac_bits=28,
        placement="blobs", mass=(0.5, 2.0), v_sigma=1.0, c_sigma=0.05,
        max_mass=2.0, max_speed=8.0, max_affine=0.5, seed=_seed(4)),
    # Full substep loop: 8M particles, dam-break block, 256^3 nodes.
    "dam_3d_256": Workload(
        name="dam_3d_256", kind="quadratic", dim=3, n=256, n_particles=1 << 23, frac_bits=32,
        placement="dam", mass=1.0, v_sigma=0.1, c_sigma=0.05,
        max_mass=1.0, max_speed=2.0, max_affine=1000.0, seed=_seed(5),
        extra={"dt": 1e-4, "gravity": (0.0, -9.8, 0.0), "sticky": 2, "substeps": 100,
               "check_every": 10}),
    # Elastic (Neo-Hookean) cube thrown at the floor: the MLS-MPM stress term
    # on top of the APIC transfer, 64^3 nodes.  rho = m / vol0 = 8 / dx^3; with
    # mu = lambda = 1e9 the wave speed sqrt((lambda + 2 mu) / rho) ~ 38 keeps
    # c dt / dx ~ 0.24.
    "jelly_3d_64": Workload(
        name="jelly_3d_64", kind="quadratic", dim=3, n=64, n_particles=8 * 16 ** 3, frac_bits=28,
        placement="jelly", mass=1.0, v_sigma=0.05, c_sigma=0.0,
        max_mass=1.0, max_speed=50.0, max_affine=1.0e4, seed=_seed(6),
        extra={"dt": 1e-4, "gravity": (0.0, -9.8, 0.0), "sticky": 2, "substeps": 60, "check_every": 10,
               "mu": 1.0e9, "lam": 1.0e9, "v0": (0.0, -3.0, 0.0)}),
    # The same elastic cube at 256^3 nodes, side 100 cells (8M particles);
    # mu = lambda = 4e9 keeps c dt / dx ~ 0.24 at rho = 8 / dx^3.
    "jelly_3d_256": Workload(
        name="jelly_3d_256", kind="quadratic", dim=3, n=256, n_particles=8 * 100 ** 3, frac_bits=28,
        placement="jelly", mass=1.0, v_sigma=0.05, c_sigma=0.0,
        max_mass=1.0, max_speed=50.0, max_affine=1.0e4, seed=_seed(7),
        extra={"dt": 1e-4, "gravity": (0.0, -9.8, 0.0), "sticky": 2, "substeps": 60, "check_every": 10,
               "mu": 4.0e9, "lam": 4.0e9, "v0": (0.0, -3.0, 0.0)}),
    # Integer-split quadratic APIC transfer (exact conservation): integer
    # positions (2^-16 cell), masses, velocities and affine entries.
    # PB-MPM (position-based MPM, elastic material): the jelly cubes, with the
    # particle state in displacement form (d = v dt for the first substep,
    # D = 0, F = I) and the iteration loop's parameters (the page's defaults: 5
    # iterations, relaxation 1.5)
    "pbmpm_jelly_3d_64": Workload(
        name="pbmpm_jelly_3d_64", kind="pbmpm", dim=3, n=64, n_particles=8 * 16 ** 3, frac_bits=32,
        placement="jelly", mass=1.0, v_sigma=0.05, c_sigma=0.0,
        max_mass=1.0, max_speed=0.5, max_affine=4.0, seed=_seed(10),
        extra={"dt": 2e-3, "gravity": (0.0, -9.8, 0.0), "band": 2, "iterations": 5, "relax": 1.5,
               "polar_iters": 12, "substeps": 20, "v0": (0.0, -3.0, 0.0)}),
    "pbmpm_jelly_3d_256": Workload(
        name="pbmpm_jelly_3d_256", kind="pbmpm", dim=3, n=256, n_particles=8 * 100 ** 3, frac_bits=32,
        placement="jelly", mass=1.0, v_sigma=0.05, c_sigma=0.0,
        max_mass=1.0, max_speed=0.5, max_affine=4.0, seed=_seed(11),
        extra={"dt": 1e-3, "gravity": (0.0, -9.8, 0.0), "band": 2, "iterations": 5, "relax": 1.5,
               "polar_iters": 12, "substeps": 10, "v0": (0.0, -3.0, 0.0)}),
    "isplit_2d_64": Workload(
        name="isplit_2d_64", kind="isplit", dim=2, n=64, n_particles=3500, frac_bits=0,
        max_mass=1000, max_speed=1000, max_affine=1000, seed=_seed(8)),
    "isplit_3d_128": Workload(
        name="isplit_3d_128", kind="isplit", dim=3, n=128, n_particles=1 << 20, frac_bits=0,
        max_mass=1000, max_speed=1000, max_affine=1000, seed=_seed(9)),
}


def scaled(w: Workload, n_particles: int, n: int | None = None) -> Workload:
    """The same workload recipe at another particle count (and grid size)."""
    return replace(w, n_particles=n_particles, n=w.n if n is None else n,
                   name=f"{w.name}@{n_particles}" + ("" if n is None else f"n{n}"))


def build(w: Workload) -> dict:
    """Materialise the workload's arrays (numpy, host memory)."""
    if w.kind == "isplit":
        return G.integer_cloud_quadratic(w.seed, w.n_particles, w.n, w.dim, int(w.max_mass), int(w.max_speed),
                                         int(w.max_affine))
    if w.kind == "cic_split":
        return G.integer_cloud(w.seed, n=w.n_particles, cells=w.n, frac_bits=w.frac_bits,
                               max_mass=int(w.max_mass), max_speed=int(w.max_speed))
    if w.placement == "pile":
        x = G.settled_pile_2d(w.seed, w.n_particles, w.n)
    elif w.placement == "dam":
        x = G.dam_break_3d(w.seed, w.n_particles, w.n)
    elif w.placement == "blobs":
        x = G.gaussian_blobs_3d(w.seed, w.n_particles, w.n)
    elif w.placement == "jelly":
        x = G.jelly_block_3d(w.seed, w.n_particles, w.n)
    elif w.placement == "uniform":
        x = 2.0 / w.n + G.uniform01(w.seed, 90, w.dim * w.n_particles).reshape(w.dim, -1) * ((w.n - 4.0) / w.n)
    else:
        raise ValueError(f"unknown placement {w.placement!r}")
    out = {"x": np.ascontiguousarray(x.astype(np.float32))}
    out.update(G.particle_fields(w.seed, w.n_particles, w.dim, w.mass, w.v_sigma, w.c_sigma))
    if w.dim == 3 and w.placement == "dam":
        dx = 1.0 / w.n
        out["vol"] = np.full(w.n_particles, dx ** 3 / 8.0, dtype=np.float32)
    if w.placement == "jelly":
        dx = 1.0 / w.n
        out["vol"] = np.full(w.n_particles, dx ** 3 / 8.0, dtype=np.float32)
        out["F"] = np.ascontiguousarray(np.tile(np.eye(3, dtype=np.float32).reshape(9, 1), (1, w.n_particles)))
        out["v"] = np.ascontiguousarray(out["v"] + np.asarray(w.extra["v0"], np.float32)[:, None])
    if w.kind == "pbmpm":
        # displacement form: v holds the displacement over the first substep
        # (velocity times dt), C the displacement gradient (zero at rest)
        out["v"] = np.ascontiguousarray(out["v"] * np.float32(w.extra["dt"]))
        out["C"] = np.zeros_like(out["C"])
    return out
