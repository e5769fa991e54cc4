"""The integer-split transfer's entry point that allocates nothing
(mpm_p2g_isplit_noalloc, the tiled path on the library's static device
scratch) against the same transfer with a caller-allocated workspace
(mpm_p2g_isplit), through the C ABI: integer arithmetic, so the grids and the
status counters must be identical.  Two calls in a row share the scratch; the
second is smaller (a different dimension, grid and particle count), so what
the first call left in the scratch must not leak into it.  Inputs past the
scratch's size are refused before any launch.
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


def device_inputs(h):
    dev = torch.device("cuda", 0)
    return tuple(torch.from_numpy(np.ascontiguousarray(h[k], dt)).to(dev)
                 for k, dt in (("X", np.int32), ("m", np.int64), ("v", np.int64), ("C", np.int64)))


def both_paths(M, dim, n, h, rng, order=None):
    """(grid, status) of the workspace call and of the no-allocation call."""
    dev = torch.device("cuda", 0)
    X, m, v, C = device_inputs(h)
    o = None if order is None else torch.from_numpy(order.astype(np.uint32).view(np.int32)).to(dev)
    out = []
    for noalloc in (False, True):
        g = torch.zeros((1 + dim,) + (n,) * dim, dtype=torch.int64, device=dev)
        st = torch.zeros(4, dtype=torch.int32, device=dev)
        if noalloc:
            M.mpm_p2g_isplit_noalloc(dim, n, X, m, v, C, o, *rng, g, st)
        else:
            ws = torch.empty(M.mpm_isplit_workspace_bytes(dim, n, m.numel()), dtype=torch.uint8, device=dev)
            M.mpm_p2g_isplit(dim, n, X, m, v, C, o, *rng, g, st, workspace=ws)
        torch.cuda.synchronize()
        out.append((g.cpu().numpy(), st.cpu().numpy().view(np.uint32)))
    return out


def test_two_calls_in_a_row_match_the_workspace_path(mpm):
    from material_point_particle_amd import _lib as L
    # first call: the 3D workload at full size (1,048,576 particles, 128^3)
    w = WORKLOADS["isplit_3d_128"]
    h = build(w)
    rng = (int(w.max_mass), int(w.max_speed), int(w.max_affine))
    assert mpm.mpm_isplit_workspace_bytes(3, w.n, w.n_particles) <= L.MPM_ISPLIT_SCRATCH_BYTES
    say("no-alloc call 1:", w.name, w.n_particles)
    (g_ws, st_ws), (g_na, st_na) = both_paths(mpm, 3, w.n, h, rng)
    assert np.array_equal(g_na, g_ws)
    assert st_na.tolist() == st_ws.tolist() == [0, 0, 0, 0]
    assert g_na[0].sum() == h["m"].sum()                      # exact conservation
    # second call, smaller: the 2D workload (3,500 particles, 64^2) in a
    # shuffled order, with a few particles outside the grid and the ranges
    w2 = WORKLOADS["isplit_2d_64"]
    h2 = build(w2)
    h2 = {k: np.array(a, copy=True) for k, a in h2.items()}
    h2["X"][0, :5] = -70000                                   # off the grid: counted in status[0]
    h2["v"][1, 5:8] = int(w2.max_speed) + 1                   # past the declared ranges: status[1]
    rng2 = (int(w2.max_mass), int(w2.max_speed), int(w2.max_affine))
    order = G.permutation(0x4D504D07 ^ 0x5F5F, 1, w2.n_particles)
    say("no-alloc call 2:", w2.name, w2.n_particles, "shuffled")
    (g_ws, st_ws), (g_na, st_na) = both_paths(mpm, 2, w2.n, h2, rng2, order=order)
    assert np.array_equal(g_na, g_ws)
    assert st_na.tolist() == st_ws.tolist() == [5, 3, 0, 0]


def test_empty_call_and_size_refusal(mpm):
    from material_point_particle_amd import _lib as L
    dev = torch.device("cuda", 0)
    g = torch.zeros((3, 8, 8), dtype=torch.int64, device=dev)
    st = torch.zeros(4, dtype=torch.int32, device=dev)
    e32 = torch.zeros((2, 0), dtype=torch.int32, device=dev)
    e64 = torch.zeros((0,), dtype=torch.int64, device=dev)
    mpm.mpm_p2g_isplit_noalloc(2, 8, e32, e64, e64, e64, None, 1, 1, 1, g, st)
    torch.cuda.synchronize()
    assert int(g.abs().sum().item()) == 0
    # 2^24 particles on 128^3 needs more than the 256 MiB scratch: refused
    np_ = 1 << 24
    assert mpm.mpm_isplit_workspace_bytes(3, 128, np_) > L.MPM_ISPLIT_SCRATCH_BYTES
    # (inputs and grid sized as a real call of this shape would be)
    m = torch.zeros(np_, dtype=torch.int64, device=dev)
    X = torch.zeros((3, np_), dtype=torch.int32, device=dev)
    v = torch.zeros((3, np_), dtype=torch.int64, device=dev)
    C = torch.zeros((9, np_), dtype=torch.int64, device=dev)
    g3 = torch.zeros((4, 128, 128, 128), dtype=torch.int64, device=dev)
    with pytest.raises(mpm.MpmError) as e:
        mpm.mpm_p2g_isplit_noalloc(3, 128, X, m, v, C, None, 1, 1, 1, g3, st)
    assert e.value.code == L.MPM_ERR_SCRATCH
