"""The full-size dam-break workload (8,388,608 particles, 256^3 nodes) in
lockstep with the oracle's own 100-substep trajectory: at substeps 0, 10, ...,
100 the particle state (x, v, C) and the P2G grid of that state must have the
SHA-256 digests the oracle's trajectory has (tests/golden/
dam_3d_256_trajectory.json, written by tests/golden/make_dam_trajectory.py,
which calls only the oracle).  An error at any substep changes every later
digest, so every substep is covered, not only the checkpoints.  Both substep
loops are checked: the separate steps (binning, P2G, restricted grid update,
G2P) and the fused resident substep (re-binned every 10 substeps).
"""
import hashlib
import json
import os
import sys

import numpy as np
import pytest
import torch

from mpm_inputs import WORKLOADS, build

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "dam_3d_256_trajectory.json")


def say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mpm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import material_point_particle_amd as M
    M.lib()
    return M


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    w = WORKLOADS[g["workload"]]
    host = {k: np.ascontiguousarray(v) for k, v in build(w).items() if k in ("x", "v", "C", "m")}
    digest = hashlib.sha256(b"".join(host[k].tobytes() for k in ("x", "v", "C", "m"))).hexdigest()
    assert digest == g["input_sha256"], "the generated inputs differ from those the golden trajectory was made from"
    return w, host, g


def sha(t) -> str:
    return hashlib.sha256(t.contiguous().cpu().numpy().tobytes()).hexdigest()


def check(cp, grid, parts, what):
    k = cp["substep"]
    if grid is not None:
        assert sha(grid) == cp["grid_sha256"], f"{what}: P2G grid of the state after substep {k}"
    if parts is not None:
        for f in ("x", "v", "C"):
            assert sha(getattr(parts, f)) == cp[f"{f}_sha256"], f"{what}: {f} after substep {k}"


@pytest.mark.timeout(900)
def test_separate_steps_follow_the_oracle_trajectory(mpm, golden):
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    w, host, g = golden
    ex = w.extra
    cps = {c["substep"]: c for c in g["checkpoints"]}
    parts = DeviceParticles(host)
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    for k in range(0, 101):
        tr.bin(parts)
        tr.p2g(parts, binned=True)                  # the P2G grid of the state after substep k
        if k in cps:
            torch.cuda.synchronize()
            say("trajectory, separate steps:", k)
            check(cps[k], tr.grid, parts, "separate steps")
        if k == 100:
            break
        tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
        tr.g2p(parts, ex["dt"])
    st = tr.status.cpu().numpy().view(np.uint32).tolist()
    assert st[3] == 0 and st[2] == g["oracle_status"][2], (st, g["oracle_status"])


@pytest.mark.timeout(900)
def test_fused_substeps_follow_the_oracle_trajectory(mpm, golden):
    from material_point_particle_amd.transfer import DeviceParticles, ResidentSubsteps, Transfer
    w, host, g = golden
    ex = w.extra
    cps = {c["substep"]: c for c in g["checkpoints"]}
    parts = DeviceParticles(host)
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    rs = ResidentSubsteps(tr, parts, ex["dt"], ex["gravity"], ex["sticky"])
    rs.start()
    torch.cuda.synchronize()
    check(cps[0], rs.grid, None, "fused substeps")
    for k in range(1, 101):
        rs.substep()                                # rs.grid: the P2G grid of the state after substep k
        if k in cps:
            rs.gather()
            torch.cuda.synchronize()
            say("trajectory, fused substeps:", k)
            check(cps[k], rs.grid, parts, "fused substeps")
            rs.rebin()
    st = tr.status.cpu().numpy().view(np.uint32).tolist()
    assert st[3] == 0 and st[2] == g["oracle_status"][2], (st, g["oracle_status"])
