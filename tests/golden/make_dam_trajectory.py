#!/usr/bin/env python3
"""Writes tests/golden/dam_3d_256_trajectory.json: SHA-256 digests of the
oracle's own 100-substep trajectory of the full-size dam-break workload
(8,388,608 particles, 256^3 nodes, 2^32, dt 1e-4, gravity -9.8 y, sticky
band 2), the workload checked against the oracle every 10 substeps.

Each substep is the oracle's P2G of the state, its grid update (consume and
zero, gravity, sticky walls) and its G2P gather and advection.  Recorded for
k = 0, 10, 20, ..., 100: digests of x, v and C after substep k and of the
P2G grid of that state (the grid substep k+1 deposits), plus the digest of
the generated inputs and the oracle's status counters.  The script calls only
the oracle (its P2G on several host threads: private grids, integer-summed,
bit-identical to the single-thread P2G) and the seeded input generator.
Run: python tests/golden/make_dam_trajectory.py  (a few minutes on 8 cores).
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mpm_inputs import WORKLOADS, build  # noqa: E402

OUT = os.path.join(HERE, "dam_3d_256_trajectory.json")
CHECKPOINTS = list(range(0, 101, 10))


def sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main():
    w = WORKLOADS["dam_3d_256"]
    ex = w.extra
    rng = (w.max_mass, w.max_speed, w.max_affine)
    state = {k: np.ascontiguousarray(v) for k, v in build(w).items() if k in ("x", "v", "C", "m")}
    threads = min(16, len(os.sched_getaffinity(0)))
    rec = {"workload": w.name, "dim": w.dim, "n": w.n, "particles": w.n_particles, "frac_bits": w.frac_bits,
           "dt": ex["dt"], "gravity": list(ex["gravity"]), "sticky": ex["sticky"],
           "ranges": list(rng), "input_sha256": sha(state["x"], state["v"], state["C"], state["m"]),
           "digest_of": "sha256 of the little-endian C-order bytes: grid int64[4][256][256][256], "
                        "x/v float32[3][n], C float32[9][n]",
           "checkpoints": []}
    status = np.zeros(4, dtype=np.int64)
    t0 = time.time()
    for k in range(0, 101):
        grid, st = oracle.p2g_quadratic_threads(w.dim, w.n, w.frac_bits, state, rng, threads)
        status += st
        if k in CHECKPOINTS:
            rec["checkpoints"].append({"substep": k, "grid_sha256": sha(grid), "x_sha256": sha(state["x"]),
                                       "v_sha256": sha(state["v"]), "C_sha256": sha(state["C"])})
            print(f"substep {k}: recorded ({time.time() - t0:.0f}s)", flush=True)
        if k == 100:
            break
        vg = oracle.grid_update(w.dim, w.n, grid, ex["dt"], ex["gravity"], ex["sticky"])
        status += oracle.g2p(w.dim, w.n, vg, state, ex["dt"])
    rec["oracle_status"] = [int(s) for s in status]
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
