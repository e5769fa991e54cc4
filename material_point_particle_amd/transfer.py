"""Device-memory driver around the C ABI: owns torch-allocated buffers and
calls the library's entry points on the current torch stream.

Every step of the transfer runs in libmpm's HIP kernels; this module only
allocates memory, copies host arrays to the device and passes pointers.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceParticles:
    """Component-major float32 particle arrays on the device."""

    def __init__(self, host: dict, device="cuda"):
        self.x = to_device(host["x"], device)
        self.v = to_device(host["v"], device)
        self.C = to_device(host["C"], device)
        self.m = to_device(host["m"], device)
        self.n = int(self.m.shape[0])

    def desc(self) -> L.mpm_particles:
        return L.particles(self.n, self.x, self.v, self.C, self.m)

    def host(self) -> dict:
        return {k: getattr(self, k).cpu().numpy() for k in ("x", "v", "C", "m")}


class ElasticParticles(DeviceParticles):
    """Particles of a Neo-Hookean solid: the APIC state plus the deformation
    gradient F[dim*dim][n] (component-major, like C), the initial volumes and
    a buffer for the stressed affine matrix C' that binning and P2G read."""

    def __init__(self, host: dict, F: np.ndarray, vol0: np.ndarray, device="cuda"):
        super().__init__(host, device)
        self.F = to_device(np.asarray(F, dtype=np.float32), device)
        self.vol0 = to_device(np.asarray(vol0, dtype=np.float32), device)
        self.C_aff = torch.empty_like(self.C)

    def affine(self) -> "StressedView":
        """The particles as P2G sees them after stress(): C replaced by C'."""
        return StressedView(self)

    def stress(self, tr: "Transfer", dt: float, mu: float, lam: float) -> None:
        L.mpm_neohookean_affine(tr.desc, self.desc(), self.F, self.vol0, dt, mu, lam, self.C_aff, tr.status)

    def update_F(self, tr: "Transfer", dt: float) -> None:
        L.mpm_update_deformation(tr.desc, self.desc(), self.F, dt)

    def update_F_stress(self, tr: "Transfer", dt: float, mu: float, lam: float) -> None:
        """update_F, then stress() for the next substep, in one pass."""
        L.mpm_update_deformation_stress(tr.desc, self.desc(), self.F, self.vol0, dt, mu, lam, self.C_aff, tr.status)

    def g2p_update_F_stress(self, tr: "Transfer", dt: float, mu: float, lam: float) -> None:
        """tr.g2p(self, dt), then update_F_stress, in one launch."""
        L.mpm_g2p_update_deformation_stress(tr.desc, tr.vg, self.desc(), dt, self.F, self.vol0, mu, lam, self.C_aff,
                                            tr.status)

    def host(self) -> dict:
        h = super().host()
        h["F"] = self.F.cpu().numpy()
        return h


class StressedView:
    def __init__(self, parts: ElasticParticles):
        self.p = parts
        self.n = parts.n

    def desc(self) -> L.mpm_particles:
        return L.particles(self.n, self.p.x, self.p.v, self.p.C_aff, self.p.m)


class Transfer:
    """One grid (dim, n, 2^frac_bits) with its binning workspace, int64
    accumulators, velocity grid and status counters."""

    def __init__(self, dim: int, n: int, frac_bits: int, ranges, n_particles: int, device="cuda"):
        self.dim, self.n, self.frac_bits = dim, n, frac_bits
        self.desc = L.grid_desc(dim, n, frac_bits)
        self.ranges = L.ranges(*ranges)
        self.n_particles = n_particles
        self.log2_bound = L.mpm_check_bounds(self.desc, n_particles, self.ranges)
        self.layout = L.mpm_workspace_layout(self.desc, n_particles)
        nbytes = self.layout.total_bytes
        self.ws = torch.empty((nbytes + 7) // 8, dtype=torch.int64, device=device)
        self.grid = torch.zeros((1 + dim,) + (n,) * dim, dtype=torch.int64, device=device)
        self.vg = torch.zeros((dim,) + (n,) * dim, dtype=torch.float32, device=device)
        self.status = torch.zeros(4, dtype=torch.int32, device=device)

    # -- steps -------------------------------------------------------------
    def bin(self, parts: DeviceParticles) -> None:
        L.mpm_bin_particles(self.desc, parts.desc(), self.ranges, self.ws, self.status)

    def p2g(self, parts: DeviceParticles, binned: bool = True, grid: torch.Tensor | None = None) -> torch.Tensor:
        g = self.grid if grid is None else grid
        L.mpm_p2g(self.desc, parts.desc(), self.ranges, self.ws if binned else None, g, self.status)
        return g

    def grid_update(self, dt: float, gravity, sticky: int, active: bool = False) -> torch.Tensor:
        """active: update only the node tiles the last binned P2G can reach
        (the workspace must hold that binning)."""
        L.mpm_grid_update(self.desc, self.ws if active else None, self.grid, self.vg, dt, gravity, sticky)
        return self.vg

    def clear(self, active: bool = False) -> None:
        """Zero the grid; active: only the node tiles the last binned P2G can
        reach (the workspace must hold that binning)."""
        L.mpm_grid_clear(self.desc, self.ws if active else None, self.grid)

    def g2p(self, parts: DeviceParticles, dt: float) -> None:
        L.mpm_g2p(self.desc, self.vg, parts.desc(), dt, self.status)

    # -- workspace views (for tests and reports) ----------------------------
    def ws_u32(self, field: str, count: int) -> torch.Tensor:
        off = getattr(self.layout, field)
        return self.ws.view(torch.int32)[off // 4: off // 4 + count]

    def meta(self) -> np.ndarray:
        return self.ws_u32("meta", 32).cpu().numpy().view(np.uint32)


class ResidentSubsteps:
    """The substep loop with the particle state kept in the binned records
    (mpm_bin_resident, mpm_g2p2g, mpm_gather_records): three grids used in
    turn, each with its node-tile flags; a substep reads grid k, deposits into
    grid k+1 and zeroes grid k-1 in the same kernel.  After start(),
    self.grid holds the deposit of the current state (the next substep's
    P2G grid)."""

    def __init__(self, tr: Transfer, parts: DeviceParticles, dt: float, gravity, sticky: int, device="cuda"):
        self.tr, self.parts = tr, parts
        self.dt, self.gravity, self.sticky = dt, list(gravity), sticky
        dim, n = tr.dim, tr.n
        self.grids = [tr.grid, torch.zeros_like(tr.grid), torch.zeros_like(tr.grid)]
        n_tiles = (n // 4) ** dim
        self.tiles = [torch.zeros(n_tiles, dtype=torch.uint8, device=device) for _ in range(3)]
        self.cur = 0

    @property
    def grid(self) -> torch.Tensor:
        return self.grids[self.cur]

    def start(self) -> None:
        """Bin the particles and deposit them into the current grid (zeroed
        here)."""
        self.grids[self.cur].zero_()
        self.tiles[self.cur].zero_()
        self.rebin()
        L.mpm_g2p2g(self.tr.desc, self.tr.ranges, self.tr.ws, self.parts.n, None, self.grids[self.cur],
                    self.tiles[self.cur], self.dt, self.gravity, self.sticky, self.tr.status)

    def rebin(self) -> None:
        L.mpm_bin_resident(self.tr.desc, self.parts.desc(), self.tr.ws, self.tr.status)

    def substep(self, stream=None) -> None:
        a, b, c = self.cur, (self.cur + 1) % 3, (self.cur + 2) % 3
        L.mpm_g2p2g(self.tr.desc, self.tr.ranges, self.tr.ws, self.parts.n, self.grids[a], self.grids[b],
                    self.tiles[b], self.dt, self.gravity, self.sticky, self.tr.status, stream,
                    grid_clear=self.grids[c], tiles_clear=self.tiles[c])
        self.cur = b

    def gather(self) -> None:
        """Write the records' x, v, C back to the particle arrays."""
        L.mpm_gather_records(self.tr.desc, self.tr.ws, self.parts.desc(), self.tr.status)


class SplitResidentSubsteps(ResidentSubsteps):
    """The resident-state substep in three launches instead of the fused
    kernel: the grid update of the node tiles the last deposit flagged
    (consuming that grid and its flags), the G2P gather over the records in
    place, and the fused kernel's deposit-only launch into the other grid.
    Two grids in turn; results identical to ResidentSubsteps'."""

    def __init__(self, tr: Transfer, parts: DeviceParticles, dt: float, gravity, sticky: int, device="cuda"):
        super().__init__(tr, parts, dt, gravity, sticky, device)
        self.grids, self.tiles = self.grids[:2], self.tiles[:2]

    def substep(self, stream=None) -> None:
        a, b = self.cur, 1 - self.cur
        tr = self.tr
        L.mpm_grid_update_tiles(tr.desc, self.grids[a], self.tiles[a], tr.vg, self.dt, self.gravity, self.sticky,
                                stream)
        L.mpm_g2p_records(tr.desc, tr.ws, self.parts.n, tr.vg, self.dt, tr.status, stream)
        L.mpm_g2p2g(tr.desc, tr.ranges, tr.ws, self.parts.n, None, self.grids[b], self.tiles[b], self.dt,
                    self.gravity, self.sticky, tr.status, stream)
        self.cur = b


class PBMPMSubsteps:
    """The position-based MPM (PB-MPM) substep of an elastic material
    ("Implementation -- GPU Optimization & Reference Codebases", section
    3.3.2) on ElasticParticles whose v holds the displacement d and whose C
    holds the displacement gradient D: `iterations` times the elastic
    projection, binning and P2G, the displacement-form grid update (into
    tr.vg) and the G2P gather (dt = 0); then the integrate step and
    F <- (I + D) F.  d and D change every iteration while x does not (beyond
    the gather's clamp, which keeps each particle in its cell): with
    `records` the particles are binned once per substep and every gather but
    the last rewrites their binned records; without it every iteration
    re-bins."""

    def __init__(self, tr: Transfer, parts: ElasticParticles, dt: float, gravity, iterations: int = 5,
                 relax: float = 1.5, polar_iters: int = 12, band: int = 2, fused: bool = True,
                 records: bool = True):
        self.tr, self.parts = tr, parts
        self.dt, self.gravity = dt, list(gravity)
        self.iterations, self.relax, self.polar_iters, self.band = iterations, relax, polar_iters, band
        self.fused = fused
        self.records = fused and records

    def project(self) -> None:
        tr, parts = self.tr, self.parts
        L.mpm_pbmpm_project_elastic(tr.desc, parts.desc(), parts.F, self.relax, self.polar_iters, tr.status)

    def deposit(self, rebin: bool = True) -> None:
        """Binning (unless the records are current), P2G and the
        displacement-form grid update of one iteration."""
        tr, parts = self.tr, self.parts
        if rebin:
            tr.bin(parts)
        tr.p2g(parts, binned=True)
        L.mpm_pbmpm_grid_update(tr.desc, tr.ws, tr.grid, tr.vg, self.band)

    def gather_project(self) -> None:
        """This iteration's G2P and the next iteration's projection in one
        pass (with `records`, the binned records rewritten too)."""
        tr, parts = self.tr, self.parts
        if self.records:
            L.mpm_pbmpm_g2p_project_records(tr.desc, tr.vg, parts.desc(), parts.F, self.relax, self.polar_iters,
                                            tr.ranges, tr.ws, tr.status)
        else:
            L.mpm_pbmpm_g2p_project(tr.desc, tr.vg, parts.desc(), parts.F, self.relax, self.polar_iters, tr.status)

    def iteration(self) -> None:
        self.project()
        self.deposit()
        self.tr.g2p(self.parts, 0.0)

    def integrate(self) -> None:
        tr, parts = self.tr, self.parts
        L.mpm_pbmpm_integrate(tr.desc, parts.desc(), self.dt, self.gravity, tr.status)
        L.mpm_update_deformation(tr.desc, parts.desc(), parts.F, 1.0)

    def gather_integrate(self) -> None:
        """The last iteration's G2P, then integrate(), in one launch."""
        tr, parts = self.tr, self.parts
        L.mpm_pbmpm_g2p_integrate(tr.desc, tr.vg, parts.desc(), parts.F, self.dt, self.gravity, tr.status)

    def substep(self) -> None:
        """fused: the first projection on its own, then every iteration's G2P
        but the last together with the next projection (with `records`, one
        binning per substep, and the last G2P with the integrate step and the F
        update); else the separate calls.  All give the same bits."""
        if self.fused:
            self.project()
            for it in range(self.iterations):
                self.deposit(rebin=it == 0 or not self.records)
                if it + 1 < self.iterations:
                    self.gather_project()
                elif self.records:
                    self.gather_integrate()
                    return
                else:
                    self.tr.g2p(self.parts, 0.0)
        else:
            for _ in range(self.iterations):
                self.iteration()
        self.integrate()
