#!/usr/bin/env python3
"""Benchmark of the MI355X P2G hot path: one JSON line on stdout.

A step is one pass of the whole hot path over the 16M-particle Gaussian-blob
workload (256^3 nodes, 4 int64 channels at 2^28): reset the accumulators
(only the node tiles the previous P2G into that grid could reach), bin the
particles into 4^3-cell tiles (counting sort), and run the tiled fixed-point
APIC P2G.  Inputs are resident in HBM before timing starts; two input copies
(each with its own workspace and grid) alternate between steps so that the
256 MB last-level cache cannot keep one step's data for the next.

Timing: HIP events recorded on the stream the library launches on (torch's
current stream), around each stage of each timed step; `value` is particles
per second of the whole step.  The `roofline` object is for the dominant
kernel, using algorithmic bytes (particle records read once, touched nodes
written once) over its average event-measured duration; `alu_roofline` puts
the same kernel against the vector-ALU issue rate (the lane operations the
fixed-order transfer needs per particle, over the same duration), which is
what limits it.  `cpu_baseline` is
the oracle (plain single-threaded C) timed on this host's cores over one
step of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
# Vector-ALU issue rates on MI355X, in lane operations per second, by instruction class:
#  - "slow" class (v_rndne_f32, v_cvt_f64_f32, v_add_f64, shifts, conversions): one 64-lane instruction per SIMD
#    every 4 cycles, 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T (the fp64 vector peak, 78.6 TFLOP/s, counts an
#    FMA as two);
#  - "fast" class (v_add_f32, v_sub_f32, v_mul_f32, v_add_u32, v_and_b32): issued faster than that; no datasheet
#    figure names the rate, so the peak taken is the measured one, 53.6 T at 4 waves per SIMD (the slow class
#    measured 31.8-35.5 T in the same run, 81-90% of its 39.3 T).
SLOW_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
FAST_PEAK_TOPS = 53.6


# Lane operations the fixed-order transfer needs per particle, however it is scheduled, by class, with every
# product or sum that several stencil nodes share counted once.  Fast class (float32 multiply and add): per axis
# 18 for the stencil (x*n, the -0.5, t = g - b, the three weight factors, squares and scalings, the three node
# offsets and their scaling by dx); m*S and the weight prefix products (m S wx) wy ... (3 + 9 + 27 in 3D); per
# velocity channel DIM products C_de r_e and the prefix sums of u (3 + 9 + 27); DIM momentum products per node.
# Slow class: per axis floor and the base cell's conversion, and per node and channel one rounding, one widening
# to float64 and three quarters of a float64 add (three adds per group of four contributions).
def alu_ops_per_particle(dim: int) -> tuple[float, float]:
    nodes = 3 ** dim
    prefixes = sum(3 ** k for k in range(1, dim + 1))
    fast = 18 * dim + (1 + prefixes) + dim * (3 * dim + prefixes) + dim * nodes
    slow = 2 * dim + (2 + 0.75) * (1 + dim) * nodes
    return fast, slow


# Algorithmic bytes per P2G (the survey's per-unit figures): each particle's state (x, v, C, m) and its index
# entry read once, each touched node's 1 + DIM int64 channels written once.
def p2g_algorithmic_bytes(dim: int, particles: int, touched: int) -> int:
    state = 4 * (2 * dim + dim * dim + 1)
    return particles * (state + 4) + touched * 8 * (1 + dim)


METRIC = "P2G particles/sec and achieved HBM GB/s (% of peak), 3D 16M particles, 1 GPU"


P2G_SOURCES = ("material_point_particle_amd/csrc/p2g.hip", "material_point_particle_amd/csrc/p2g_device.hpp",
               "material_point_particle_amd/csrc/common.hpp")
ISPLIT_SOURCES = ("material_point_particle_amd/csrc/isplit.hip", "material_point_particle_amd/csrc/common.hpp")


def profile_record(name: str = "p2g_tiled_blobs_3d_256", sources: tuple = P2G_SOURCES):
    """The machine-readable record of a committed rocprofv3 summary (the last
    JSON block of profiles/<name>.md: counter-derived bytes, instruction
    counts, limiter), or None when the kernel's sources changed since the
    counters were taken (their SHA-256 no longer matches the record's)."""
    import hashlib
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    try:
        text = open(os.path.join(here, "profiles", name + ".md")).read()
        rec = json.loads(re.findall(r"```json\n(.*?)\n```", text, re.S)[-1])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources_sha256_16") != h.hexdigest()[:16]:
        return None
    return rec


def stage_stats(ms: np.ndarray) -> dict:
    """Mean, median, p10 and p90 of per-step times (ms)."""
    return {"mean": round(float(ms.mean()), 4), "median": round(float(np.median(ms)), 4),
            "p10": round(float(np.percentile(ms, 10)), 4), "p90": round(float(np.percentile(ms, 90)), 4)}


def time_copy(torch, gib: float = 1.0, reps: int = 10) -> dict:
    """Device-to-device copy of `gib` GiB timed with HIP events: the practical
    HBM ceiling (bytes read + written per second), median over reps."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    t = float(np.median(ms))
    return {"bytes": 2 * n * 4, "ms": round(t, 4), "gbs": round(2 * n * 4 / (t * 1e-3) / 1e9, 1)}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measure_substeps(args, torch, w, build, DeviceParticles, Transfer):
    """The full MPM substep on the 8M-particle dam-break workload (256^3 nodes,
    2^32): binning, tiled P2G, grid update (consume-and-zero, gravity, sticky
    walls; restricted to the node tiles the P2G can reach) and APIC G2P with
    advection, substep after substep on the evolving state, timed per stage
    with HIP events on the library's stream."""
    host = build(w)
    ex = w.extra
    parts = DeviceParticles(host)
    del host
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    stream = torch.cuda.current_stream()

    def substep(ev=None):
        if ev:
            ev[0].record(stream)
        tr.bin(parts)
        if ev:
            ev[1].record(stream)
        tr.p2g(parts, binned=True)
        if ev:
            ev[2].record(stream)
        tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
        if ev:
            ev[3].record(stream)
        tr.g2p(parts, ex["dt"])
        if ev:
            ev[4].record(stream)

    for _ in range(3):
        substep()
    torch.cuda.synchronize()
    k = args.substeps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(k)]
    for i in range(k):
        substep(events[i])
    torch.cuda.synchronize()
    st = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in events]).mean(axis=0)
    ms = float(st.sum())
    bin_ms, p2g_ms, upd_ms, g2p_ms = (float(v) for v in st)
    # workload facts for the algorithmic byte counts, from one more binning and
    # P2G of the current state (then consumed by a grid update)
    tr.bin(parts)
    tr.p2g(parts, binned=True)
    torch.cuda.synchronize()
    nz = tr.grid != 0
    touched = int(nz.any(dim=0).sum().item())
    with_mass = int(nz[0].sum().item())
    meta = tr.meta()
    tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True)
    torch.cuda.synchronize()
    lay = tr.layout
    active_nodes = int(tr.ws.view(torch.uint8)[lay.tile_active: lay.tile_active + lay.n_tiles].sum().item()) * 4 ** w.dim
    # grid update: read M and zero M, P, write v at every reachable node; read P where M != 0
    upd_bytes = active_nodes * (8 + 8 * (1 + w.dim) + 4 * w.dim) + with_mass * 8 * w.dim
    g2p_bytes = parts.n * (4 * w.dim + 4 * (2 * w.dim + w.dim * w.dim)) + touched * 4 * w.dim
    rec_bytes = 4 * (2 * w.dim + w.dim * w.dim + 1)
    p2g_bytes = int(meta[2]) * rec_bytes + touched * 8 * (1 + w.dim)
    status = tr.status.cpu().numpy().view(np.uint32).tolist()
    log(f"substeps: {ms:.3f} ms (bin {bin_ms:.3f}, p2g {p2g_ms:.3f}, grid update {upd_ms:.3f}, g2p {g2p_ms:.3f})")

    def gbs(b, t):
        return round(b / (t * 1e-3) / 1e9, 1)

    return {
        "workload": f"{w.name}: {parts.n} particles, dam-break block, {w.n}^3 nodes, {1 + w.dim} int64 channels at "
                    f"2^{w.frac_bits}, dt {ex['dt']}, gravity {ex['gravity'][1]}, sticky band {ex['sticky']}",
        "substeps": k, "ms_per_substep": round(ms, 4), "particles_per_s": round(parts.n / (ms * 1e-3), 1),
        "stages_ms": {"bin": round(bin_ms, 4), "p2g": round(p2g_ms, 4), "grid_update": round(upd_ms, 4),
                      "g2p": round(g2p_ms, 4)},
        "grid_update": {"bound": "hbm", "bytes": upd_bytes, "achieved_gbs": gbs(upd_bytes, upd_ms),
                        "frac": round(gbs(upd_bytes, upd_ms) / HBM_PEAK_GBS, 4), "reachable_nodes": active_nodes,
                        "nodes_with_mass": with_mass},
        "g2p": {"bound": "hbm", "bytes": g2p_bytes, "achieved_gbs": gbs(g2p_bytes, g2p_ms),
                "frac": round(gbs(g2p_bytes, g2p_ms) / HBM_PEAK_GBS, 4)},
        "p2g": {"bound": "hbm", "bytes": p2g_bytes, "achieved_gbs": gbs(p2g_bytes, p2g_ms),
                "frac": round(gbs(p2g_bytes, p2g_ms) / HBM_PEAK_GBS, 4)},
        "status": status,
    }


def measure_fused(args, torch, w, build, DeviceParticles, Transfer, split=False):
    """The dam-break substep with the particle state resident in the binned
    records (8M particles, 256^3 nodes), re-binned every 10 substeps (gather
    of the records into the particle arrays and a resident binning), all
    inside the timed region.  The fused form: one G2P2G kernel per substep
    (grid update on load, gather and advection, deposit into the next of
    three grids, and the clear of the grid read in the previous substep).
    split: three launches per substep over two grids (grid update of the node
    tiles the last deposit flagged, consuming them; G2P over the records in
    place; the deposit), each timed with events."""
    from material_point_particle_amd.transfer import ResidentSubsteps, SplitResidentSubsteps
    import material_point_particle_amd._lib as L
    host = build(w)
    ex = w.extra
    parts = DeviceParticles(host)
    del host
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    rs = (SplitResidentSubsteps if split else ResidentSubsteps)(tr, parts, ex["dt"], ex["gravity"], ex["sticky"])
    stream = torch.cuda.current_stream()
    every = 10
    rs.start()
    for _ in range(3):
        rs.substep()
    torch.cuda.synchronize()
    k = args.substeps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(k)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(k):
        e = ev[i]
        e[0].record(stream)
        if split:
            a, b = rs.cur, 1 - rs.cur
            L.mpm_grid_update_tiles(tr.desc, rs.grids[a], rs.tiles[a], tr.vg, rs.dt, rs.gravity, rs.sticky, stream)
            e[1].record(stream)
            L.mpm_g2p_records(tr.desc, tr.ws, parts.n, tr.vg, rs.dt, tr.status, stream)
            e[2].record(stream)
            L.mpm_g2p2g(tr.desc, tr.ranges, tr.ws, parts.n, None, rs.grids[b], rs.tiles[b], rs.dt, rs.gravity,
                        rs.sticky, tr.status, stream)
            rs.cur = b
        else:
            rs.substep(stream)
            e[1].record(stream)
            e[2].record(stream)
        e[3].record(stream)
        if (i + 1) % every == 0:
            rs.gather()
            rs.rebin()
        e[4].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(stop) / k
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev])
    rebin_ms = st[:, 3].sum() / max(1, k // every)
    status = tr.status.cpu().numpy().view(np.uint32).tolist()
    if split:
        stages = {"grid_update_tiles": round(float(st[:, 0].mean()), 4), "g2p_records": round(float(st[:, 1].mean()), 4),
                  "deposit": round(float(st[:, 2].mean()), 4), "rebin_each": round(float(rebin_ms), 4)}
        log(f"split resident substeps: {total:.3f} ms (grid update {stages['grid_update_tiles']:.3f}, g2p over the "
            f"records {stages['g2p_records']:.3f}, deposit {stages['deposit']:.3f}, re-bin {rebin_ms:.3f} every {every})")
    else:
        stages = {"g2p2g": round(float(st[:, 0].mean()), 4), "rebin_each": round(float(rebin_ms), 4)}
        log(f"fused substeps: {total:.3f} ms (g2p2g with the third grid's clear {stages['g2p2g']:.3f}, re-bin "
            f"{rebin_ms:.3f} every {every})")
    return {
        "workload": f"{w.name}: {parts.n} particles, dam-break block, {w.n}^3 nodes, state resident in the binned "
                    f"records, re-binned every {every} substeps" + (", three launches per substep over two grids"
                                                                    if split else ", one fused kernel per substep"),
        "substeps": k, "ms_per_substep": round(total, 4), "particles_per_s": round(parts.n / (total * 1e-3), 1),
        "stages_ms": stages,
        "status": status,
    }


def measure_elastic(args, torch, w, build, Transfer):
    """The elastic substep (MLS-MPM with the Neo-Hookean stress term) on the
    8M-particle jelly cube at 256^3 nodes: binning, P2G with the stressed
    affine matrix, restricted grid update, then G2P with the deformation-gradient
    update and the next substep's stressed affine matrix in one launch (the
    first substep's stress is its own call, before the warm-up), substep after
    substep on the evolving state, timed per stage with HIP events; then G2P
    and the pass after it as two launches, once, for their separate times.
    Algorithmic bytes of the fused elementwise pass: C, F, m, vol0 read and F,
    C' written (152 B per particle; the two separate passes move 116 + 108 B)."""
    from material_point_particle_amd.transfer import ElasticParticles
    host = build(w)
    ex = w.extra
    parts = ElasticParticles(host, host["F"], host["vol"])
    del host
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    stream = torch.cuda.current_stream()

    def substep(ev=None):
        steps = (lambda: tr.bin(parts.affine()),
                 lambda: tr.p2g(parts.affine(), binned=True),
                 lambda: tr.grid_update(ex["dt"], ex["gravity"], ex["sticky"], active=True),
                 lambda: parts.g2p_update_F_stress(tr, ex["dt"], ex["mu"], ex["lam"]))
        for i, f in enumerate(steps):
            if ev:
                ev[i].record(stream)
            f()
        if ev:
            ev[len(steps)].record(stream)

    parts.stress(tr, ex["dt"], ex["mu"], ex["lam"])
    for _ in range(3):
        substep()
    torch.cuda.synchronize()
    k = args.substeps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(k)]
    for i in range(k):
        substep(events[i])
    torch.cuda.synchronize()
    st = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in events]).mean(axis=0)
    ms = float(st.sum())
    names = ("bin", "p2g", "grid_update", "g2p_update_F_stress")
    status = tr.status.cpu().numpy().view(np.uint32).tolist()
    log(f"elastic substeps: {ms:.3f} ms (" + ", ".join(f"{n} {t:.3f}" for n, t in zip(names, st)) + ")")

    def gbs(b, t):
        return round(b / (t * 1e-3) / 1e9, 1)

    # the pass after the gather, timed alone for its HBM rate (the same kernel
    # as the second loop of the one-launch call), and G2P on its own
    reps = 5
    sep = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in sep:
        e[0].record(stream)
        tr.g2p(parts, ex["dt"])
        e[1].record(stream)
        parts.update_F_stress(tr, ex["dt"], ex["mu"], ex["lam"])
        e[2].record(stream)
    torch.cuda.synchronize()
    g2p_ms = sum(e[0].elapsed_time(e[1]) for e in sep) / reps
    fs_ms = sum(e[1].elapsed_time(e[2]) for e in sep) / reps
    log(f"elastic: as two launches G2P {g2p_ms:.3f} + F update with stress {fs_ms:.3f} ms")
    f_bytes = parts.n * 152
    return {
        "workload": f"{w.name}: {parts.n} particles, Neo-Hookean cube (mu {ex['mu']:g}, lambda {ex['lam']:g}) "
                    f"thrown at the floor, {w.n}^3 nodes, 2^{w.frac_bits}, dt {ex['dt']}",
        "substeps": k, "ms_per_substep": round(ms, 4), "particles_per_s": round(parts.n / (ms * 1e-3), 1),
        "stages_ms": {n: round(float(t), 4) for n, t in zip(names, st)},
        "two_launches_ms": {"g2p": round(g2p_ms, 4), "update_F_stress": round(fs_ms, 4)},
        "update_F_stress": {"bound": "hbm", "bytes": f_bytes, "achieved_gbs": gbs(f_bytes, fs_ms),
                            "frac": round(gbs(f_bytes, fs_ms) / HBM_PEAK_GBS, 4)},
        "status": status,
    }


def measure_pbmpm(args, torch, w, build):
    """The position-based MPM substep (elastic material) on the 8M-particle
    jelly cube at 256^3: per substep 5 iterations of P2G, displacement-form
    grid update and G2P gather, each iteration opened by the elastic
    projection (the first on its own, the others in the previous iteration's
    gather pass), then the integrate step and F <- (I + D) F, timed per stage
    with HIP events over the evolving state.  The particles are binned once per
    substep, after the first projection; every gather but the last rewrites
    their binned records (mpm_pbmpm_g2p_project_records).  The same loop
    re-binning every iteration (mpm_pbmpm_g2p_project) is timed after it, from
    the same starting state, for comparison.  The projection is float64 ALU work (108 B per particle: F and
    D read, D written); the integrate step reads and writes x and d (48 B)."""
    import material_point_particle_amd._lib as L
    from material_point_particle_amd.transfer import ElasticParticles, PBMPMSubsteps, Transfer
    host = build(w)
    ex = w.extra
    parts = ElasticParticles(host, host["F"], host["vol"])
    del host
    tr = Transfer(w.dim, w.n, w.frac_bits, (w.max_mass, w.max_speed, w.max_affine), parts.n)
    loop = PBMPMSubsteps(tr, parts, ex["dt"], ex["gravity"], ex["iterations"], ex["relax"], ex["polar_iters"],
                         ex["band"])
    stream = torch.cuda.current_stream()
    names = ("project", "bin", "p2g", "grid_update", "g2p_project", "g2p", "g2p_integrate")
    calls = {"project": loop.project,
             "bin": lambda: tr.bin(parts),
             "p2g": lambda: tr.p2g(parts, binned=True),
             "grid_update": lambda: L.mpm_pbmpm_grid_update(tr.desc, tr.ws, tr.grid, tr.vg, loop.band),
             "g2p_project": loop.gather_project,
             "g2p": lambda: tr.g2p(parts, 0.0),
             "g2p_integrate": loop.gather_integrate}
    last = loop.iterations - 1

    def stage_order():
        order = ["project"]
        for it in range(loop.iterations):
            if it == 0 or not loop.records:
                order.append("bin")
            order += ["p2g", "grid_update"]
            order.append("g2p_project" if it < last else ("g2p_integrate" if loop.records else "g2p"))
        return order

    order = stage_order()

    def substep(ev=None):
        for i, nm in enumerate(order):
            if ev:
                ev[i].record(stream)
            calls[nm]()
        if ev:
            ev[len(order)].record(stream)
        if order[-1] != "g2p_integrate":
            loop.integrate()
        if ev:
            ev[len(order) + 1].record(stream)

    def timed(k):
        """k substeps after one untimed: the mean substep and per-stage times."""
        substep()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 2)] for _ in range(k)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(k):
            substep(events[i])
        stop.record(stream)
        torch.cuda.synchronize()
        st = dict.fromkeys(names, 0.0)
        integ = 0.0
        for ev in events:
            for i, nm in enumerate(order):
                st[nm] += ev[i].elapsed_time(ev[i + 1])
            integ += ev[len(order)].elapsed_time(ev[len(order) + 1])
        return start.elapsed_time(stop) / k, {nm: t / k for nm, t in st.items() if nm in order}, integ / k

    k = max(3, args.substeps // 4)
    start_state = [t.clone() for t in (parts.x, parts.v, parts.C, parts.F)]
    total, st, integ = timed(k)
    status = tr.status.cpu().numpy().view(np.uint32).tolist()
    log(f"pbmpm substeps: {total:.3f} ms (" + ", ".join(f"{nm} {t:.3f}" for nm, t in st.items()) +
        f", integrate {integ:.3f}; {loop.iterations} iterations, {order.count('bin')} binning)")
    # the same loop re-binning every iteration, from the same state
    total_rebin, st_rebin = None, {}
    if not getattr(args, "no_pbmpm_rebin", False):
        for t, t0 in zip((parts.x, parts.v, parts.C, parts.F), start_state):
            t.copy_(t0)
        loop.records = False
        order = stage_order()
        total_rebin, st_rebin, _ = timed(k)
        loop.records = True
        log(f"pbmpm substeps re-binning every iteration: {total_rebin:.3f} ms (" +
            ", ".join(f"{nm} {t:.3f}" for nm, t in st_rebin.items()) + ")")
    del start_state

    def gbs(b, t):
        return round(b / (t * 1e-3) / 1e9, 1)

    proj_ms = st["project"]
    return {
        "workload": f"{w.name}: {parts.n} particles, elastic cube falling onto the floor, {w.n}^3 nodes, "
                    f"2^{w.frac_bits}, dt {ex['dt']}, {loop.iterations} iterations per substep, relaxation "
                    f"{loop.relax}, {loop.polar_iters} Newton polar steps, guardian band {loop.band}",
        "substeps": k, "ms_per_substep": round(total, 4), "particles_per_s": round(parts.n / (total * 1e-3), 1),
        "stages_ms_per_substep": {nm: round(float(t), 4) for nm, t in st.items()},
        "integrate_ms": round(float(integ), 4),
        "project": {"bytes": parts.n * 108, "ms_per_call": round(float(proj_ms), 4),
                    "achieved_gbs": gbs(parts.n * 108, proj_ms), "bound": "alu (float64 Newton polar iteration)"},
        "g2p_project_ms_per_call": round(float(st["g2p_project"]) / last, 4) if last > 0 else None,
        "binnings_per_substep": 1,
        "ms_per_substep_rebinning_every_iteration": round(total_rebin, 4) if total_rebin else None,
        "stages_ms_per_substep_rebinning_every_iteration": {nm: round(float(t), 4) for nm, t in st_rebin.items()},
        "status": status,
    }


def measure_isplit(args, torch, w, build):
    """The integer-split quadratic APIC transfer (exact conservation) on
    1,048,576 integer particles at 128^3 nodes, one mpm_p2g_isplit call per
    launch accumulating into one grid, timed with HIP events: the tiled path
    (counting sort into 8^3-cell tiles, on-chip node blocks) and the direct
    path (27 x 4 int64 global atomics per particle).  Per particle a call
    reads 116 B (X int32 x3, m, v x3, C x9 int64)."""
    import material_point_particle_amd as M
    host = build(w)
    dev = torch.device("cuda", 0)
    X = torch.from_numpy(host["X"]).to(dev)
    m = torch.from_numpy(host["m"]).to(dev)
    v = torch.from_numpy(host["v"]).to(dev)
    C = torch.from_numpy(host["C"]).to(dev)
    grid = torch.zeros((1 + w.dim,) + (w.n,) * w.dim, dtype=torch.int64, device=dev)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    ws = torch.empty(M.mpm_isplit_workspace_bytes(w.dim, w.n, w.n_particles), dtype=torch.uint8, device=dev)
    rng = (int(w.max_mass), int(w.max_speed), int(w.max_affine))
    stream = torch.cuda.current_stream()
    np_ = w.n_particles

    def timed(workspace, k):
        def launch():
            M.mpm_p2g_isplit(w.dim, w.n, X, m, v, C, None, *rng, grid, status, workspace=workspace)
        for _ in range(2):
            launch()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
        ev[0].record(stream)
        for i in range(k):
            launch()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(k)]))

    k = max(5, args.substeps)
    ms_t = timed(ws, k)
    ms_d = timed(None, 5)
    atomics = np_ * 27 * (1 + w.dim)
    rd = np_ * 116
    # the accumulating kernel against the VALU issue rate: its issued lane-ops
    # per particle and its own duration come from the committed counter
    # record (null once its sources change); the rounded products per second
    # of the whole call are measured here
    splits = (1 + w.dim * (1 + w.dim)) * sum(3 ** k_ for k_ in range(w.dim))
    rec = profile_record("isplit_tiled_isplit_3d_128", ISPLIT_SOURCES)
    alu = {"bound": "alu", "kernel": "is_tiled_kernel<3, true>", "unit": "T lane-ops/s",
           "peak": round(SLOW_PEAK_TOPS, 2),
           "peak_basis": "one 64-lane VALU instruction per SIMD every 4 cycles (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz)",
           "splits_per_particle": splits, "rounded_products_per_particle": 2 * splits,
           "rounded_products_per_s_whole_call": round(2 * splits * np_ / (ms_t * 1e-3), 1),
           "achieved": None, "frac": None, "lane_ops_per_particle": None, "kernel_ms": None, "valu_busy": None}
    if rec is not None:
        achieved = rec["valu_lane_ops_per_particle"] * np_ / (rec["kernel_us"] * 1e-6) / 1e12
        alu.update({"achieved": round(achieved, 2), "frac": round(achieved / SLOW_PEAK_TOPS, 4),
                    "lane_ops_per_particle": rec["valu_lane_ops_per_particle"],
                    "kernel_ms": round(rec["kernel_us"] * 1e-3, 4), "valu_busy": rec["valu_busy"]})
    log(f"isplit: tiled {ms_t:.3f} ms, direct {ms_d:.3f} ms per call ({np_ / (ms_t * 1e-3) / 1e9:.2f} G particles/s)")
    return {
        "workload": f"{w.name}: {np_} integer particles uniform over {w.n}^3 nodes, |m|,|v|,|C| <= "
                    f"{rng[0]}, 2^-16 cell positions",
        "calls": k, "ms_per_call": round(ms_t, 4), "particles_per_s": round(np_ / (ms_t * 1e-3), 1),
        "read_bytes_per_call": rd, "read_gbs": round(rd / (ms_t * 1e-3) / 1e9, 1),
        "alu_roofline": alu,
        "direct": {"ms_per_call": round(ms_d, 4), "particles_per_s": round(np_ / (ms_d * 1e-3), 1),
                   "atomics_per_call": atomics, "atomics_per_s": round(atomics / (ms_d * 1e-3), 1)},
        "status": status.cpu().numpy().view(np.uint32).tolist(),
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="blobs_3d_256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="particles in the CPU-baseline sample (0: all)")
    ap.add_argument("--no-shuffled", action="store_true",
                    help="skip the headline step on the shuffled particle order (profiling runs)")
    ap.add_argument("--no-substep", action="store_true",
                    help="skip the full-substep measurement (binning, P2G, grid update, G2P) on the dam-break workload")
    ap.add_argument("--substeps", type=int, default=20, help="timed substeps of the full-substep measurement")
    ap.add_argument("--only-substep", action="store_true",
                    help="run only the full-substep measurement (for profiling it alone); prints its object")
    ap.add_argument("--no-elastic", action="store_true",
                    help="skip the elastic-substep measurement (Neo-Hookean stress term) on the jelly cube")
    ap.add_argument("--only-elastic", action="store_true",
                    help="run only the elastic-substep measurement; prints its object")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-substep measurement (state resident in the binned records)")
    ap.add_argument("--only-fused", action="store_true",
                    help="run only the fused-substep measurement; prints its object")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the split resident substep (grid update of flagged tiles, G2P over records, deposit)")
    ap.add_argument("--only-split", action="store_true",
                    help="run only the split resident substep measurement; prints its object")
    ap.add_argument("--no-pbmpm", action="store_true",
                    help="skip the position-based MPM substep measurement on the jelly cube")
    ap.add_argument("--only-pbmpm", action="store_true",
                    help="run only the position-based MPM substep measurement; prints its object")
    ap.add_argument("--no-pbmpm-rebin", action="store_true",
                    help="skip the PB-MPM comparison loop that re-bins every iteration (profiling runs)")
    ap.add_argument("--no-isplit", action="store_true",
                    help="skip the integer-split quadratic transfer measurement")
    ap.add_argument("--only-isplit", action="store_true",
                    help="run only the integer-split quadratic transfer measurement; prints its object")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the hot path is measured on "
              "one GPU's share at its real shape)", file=sys.stderr)
        sys.exit(2)

    import torch

    import material_point_particle_amd as M
    from material_point_particle_amd.transfer import DeviceParticles, Transfer
    from mpm_inputs import WORKLOADS, build

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    M.lib()
    if args.only_fused:
        print(json.dumps({"substep_fused": measure_fused(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles,
                                                         Transfer)}), flush=True)
        return
    if args.only_split:
        print(json.dumps({"substep_split": measure_fused(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles,
                                                         Transfer, split=True)}), flush=True)
        return
    if args.only_pbmpm:
        print(json.dumps({"pbmpm": measure_pbmpm(args, torch, WORKLOADS["pbmpm_jelly_3d_256"], build)}), flush=True)
        return
    if args.only_isplit:
        print(json.dumps({"isplit": measure_isplit(args, torch, WORKLOADS["isplit_3d_128"], build)}), flush=True)
        return
    if args.only_elastic:
        print(json.dumps({"elastic": measure_elastic(args, torch, WORKLOADS["jelly_3d_256"], build, Transfer)}),
              flush=True)
        return
    if args.only_substep:
        print(json.dumps({"substep": measure_substeps(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles,
                                                      Transfer)}), flush=True)
        return
    w = WORKLOADS[args.workload]
    rng = (w.max_mass, w.max_speed, w.max_affine)
    t0 = time.time()
    host = build(w)
    log(f"inputs {w.name}: {w.n_particles} particles in {time.time() - t0:.1f}s")
    stream = torch.cuda.current_stream()

    def run_steps(h, steps, warmup, label):
        """Two device copies of the inputs, each with its own workspace and
        grid, stepped alternately: per-step (reset, binning, P2G) event times,
        whole-run time, and the first copy's grid and bins afterwards."""
        copies = []
        for _ in range(2):
            parts = DeviceParticles(h)
            copies.append((parts, Transfer(w.dim, w.n, w.frac_bits, rng, parts.n)))
        torch.cuda.synchronize()

        def step(k, ev=None):
            parts, tr = copies[k % 2]
            if ev:
                ev[0].record(stream)
            # reset: the node tiles this copy's previous P2G reached (its bins
            # are still in the workspace); the first step of a copy clears all
            tr.clear(active=k >= 2)
            if ev:
                ev[1].record(stream)
            tr.bin(parts)
            if ev:
                ev[2].record(stream)
            tr.p2g(parts, binned=True)
            if ev:
                ev[3].record(stream)

        for k in range(warmup):
            step(k)
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            step(warmup + k, events[k])
        stop.record(stream)
        torch.cuda.synchronize()
        total = start.elapsed_time(stop)
        stages = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in events])
        log(f"{label}: {steps} steps, {total / steps:.3f} ms/step (median reset {np.median(stages[:, 0]):.3f}, "
            f"binning {np.median(stages[:, 1]):.3f}, p2g {np.median(stages[:, 2]):.3f})")
        return total, stages, copies

    total_ms, stage, copies = run_steps(host, args.steps, args.warmup, "timed (generator order)")
    ms_step = total_ms / args.steps
    clear_ms, bin_ms, p2g_ms = stage.mean(axis=0)

    # workload facts for the algorithmic byte counts
    parts, tr = copies[0]
    meta = tr.meta()
    binned = int(meta[2])
    runs, keys = int(meta[6]), int(meta[7])
    touched = int((tr.grid != 0).any(dim=0).sum().item())
    status = tr.status.cpu().numpy().view(np.uint32).tolist()
    rec_bytes = 4 * (2 * w.dim + w.dim * w.dim + 1)          # x, v, C, m
    p2g_bytes = p2g_algorithmic_bytes(w.dim, binned, touched)
    bin_bytes = binned * (rec_bytes + rec_bytes + 4)           # read particles, write records and the index
    p2g_gbs = p2g_bytes / (p2g_ms * 1e-3) / 1e9
    bin_gbs = bin_bytes / (bin_ms * 1e-3) / 1e9
    del copies, parts, tr
    torch.cuda.empty_cache()

    # the same step on the same particles in a seeded shuffled order: binning
    # sees every chunk spread over the blobs' tiles instead of a few
    shuffled = None
    if not args.no_shuffled:
        from mpm_inputs import generators as G
        perm = G.permutation(w.seed ^ 0x5F5F, 0x5EED, w.n_particles)
        shuffled_host = {k: np.ascontiguousarray(v[..., perm]) for k, v in host.items()}
        sh_total, sh_stage, sh_copies = run_steps(shuffled_host, args.steps, args.warmup, "timed (shuffled order)")
        sh_meta = sh_copies[0][1].meta()
        sh_runs, sh_keys = int(sh_meta[6]), int(sh_meta[7])
        del sh_copies, shuffled_host
        torch.cuda.empty_cache()
        sh_ms = sh_total / args.steps
        shuffled = {
            "order": "the same particles in a seeded random order",
            "ms_per_step": round(sh_ms, 4), "particles_per_s": round(w.n_particles / (sh_ms * 1e-3), 1),
            "ratio_to_generator_order": round(sh_ms / ms_step, 4),
            "binning_runs": sh_runs, "mean_run": round(binned / max(sh_runs, 1), 1),
            "cell_keys_written": bool(sh_keys),
            "stages_ms": {"reset": stage_stats(sh_stage[:, 0]), "binning": stage_stats(sh_stage[:, 1]),
                          "p2g": stage_stats(sh_stage[:, 2])},
        }

    copy = time_copy(torch)
    log(f"device copy: {copy['gbs']} GB/s (read + write)")

    # The metric is the P2G kernel's particle rate and achieved HBM bandwidth, so the roofline object is the
    # P2G kernel's (timed per launch with events around mpm_p2g).  Binning is reported beside it.
    rec = profile_record()
    roofline = {"bound": "hbm", "achieved": round(p2g_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(p2g_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if rec is None else int(rec["hbm_read_bytes"] + rec["hbm_write_bytes"]),
                "kernel": "p2g_tiled_kernel<3>", "bytes_per_launch": int(p2g_bytes),
                "bytes_per_unit": {"particle": rec_bytes + 4, "touched_node": 8 * (1 + w.dim)},
                "ms_per_launch": round(float(p2g_ms), 4),
                "copy_gbs": copy["gbs"], "frac_of_copy": round(p2g_gbs / copy["gbs"], 4),
                "limiter": None if rec is None else rec.get("limiter")}
    # the same kernel against the vector-ALU issue rates of the instruction classes it needs
    fast, slow = alu_ops_per_particle(w.dim)
    floor_s = binned * (fast / (FAST_PEAK_TOPS * 1e12) + slow / (SLOW_PEAK_TOPS * 1e12))
    ops = fast + slow
    peak = ops * binned / floor_s / 1e12
    alu_tops = ops * binned / (p2g_ms * 1e-3) / 1e12
    alu = {"bound": "alu", "achieved": round(alu_tops, 2), "peak": round(peak, 2), "unit": "T lane-ops/s",
           "frac": round(alu_tops / peak, 4), "ops_per_particle": {"fast": fast, "slow": slow},
           "class_peaks_tops": {"fast": FAST_PEAK_TOPS, "slow": round(SLOW_PEAK_TOPS, 2)},
           "floor_ms": round(floor_s * 1e3, 4), "kernel": roofline["kernel"]}

    value = w.n_particles / (ms_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32/i64",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.n_particles} particles, 32 Gaussian blobs (sigma 4 cells), "
                               f"{w.n}^3 nodes, {1 + w.dim} int64 channels at 2^{w.frac_bits}; step = grid reset (reached tiles) + "
                               "binning into 4^3-cell tiles + tiled P2G",
                   "particles": w.n_particles, "nodes": w.n ** w.dim, "touched_nodes": touched},
        "roofline": roofline,
        "alu_roofline": alu,
        "breakdown": {
            "clear_ms": round(float(clear_ms), 4), "bin_ms": round(float(bin_ms), 4), "p2g_ms": round(float(p2g_ms), 4),
            "stages_ms": {"reset": stage_stats(stage[:, 0]), "binning": stage_stats(stage[:, 1]),
                          "p2g": stage_stats(stage[:, 2])},
            "p2g_particles_per_s": round(binned / (p2g_ms * 1e-3), 1), "p2g_gbs": round(p2g_gbs, 1),
            "p2g_frac_hbm": round(p2g_gbs / HBM_PEAK_GBS, 4), "bin_gbs": round(bin_gbs, 1),
            "bin_frac_hbm": round(bin_gbs / HBM_PEAK_GBS, 4), "bin_frac_copy": round(bin_gbs / copy["gbs"], 4),
            "bin_bytes": int(bin_bytes), "p2g_bytes": int(p2g_bytes), "status": status,
            "binning_runs": runs, "mean_run": round(binned / max(runs, 1), 1), "cell_keys_written": bool(keys),
        },
        "shuffled": shuffled,
        "copy_reference": copy,
    }

    if not args.no_substep:
        out["substep"] = measure_substeps(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles, Transfer)
        torch.cuda.empty_cache()
    if not args.no_fused:
        out["substep_fused"] = measure_fused(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles, Transfer)
        torch.cuda.empty_cache()
    if not args.no_split:
        out["substep_split"] = measure_fused(args, torch, WORKLOADS["dam_3d_256"], build, DeviceParticles, Transfer,
                                             split=True)
        torch.cuda.empty_cache()
    if not args.no_elastic:
        out["elastic"] = measure_elastic(args, torch, WORKLOADS["jelly_3d_256"], build, Transfer)
        torch.cuda.empty_cache()
    if not args.no_pbmpm:
        out["pbmpm"] = measure_pbmpm(args, torch, WORKLOADS["pbmpm_jelly_3d_256"], build)
        torch.cuda.empty_cache()
    if not args.no_isplit:
        out["isplit"] = measure_isplit(args, torch, WORKLOADS["isplit_3d_128"], build)

    if not args.no_cpu_baseline:
        # The oracle's P2G (plain C, the parity reference) on this host: once on
        # one core, once on the host's cores (the same arithmetic on contiguous
        # particle ranges with private int64 grids, integer-summed: asserted
        # bit-identical to the one-core grid).  The CPU transfer needs no
        # binning, so the sample is the transfer alone, over the first n_s
        # particles of the workload.
        import oracle
        oracle.build(force=False)
        n_s = args.cpu_sample or w.n_particles
        sample = {k: np.ascontiguousarray(v[..., :n_s]) for k, v in host.items() if k in ("x", "v", "C", "m")}
        threads = min(16, len(os.sched_getaffinity(0)))
        runs = 3
        log(f"cpu baseline on {n_s} particles: 1 thread, then {threads}, {runs} runs each")
        t1, tt = [], []
        for _ in range(runs):
            t = time.perf_counter()
            g1, s1 = oracle.p2g_quadratic(w.dim, w.n, w.frac_bits, sample, rng)
            t1.append(time.perf_counter() - t)
            t = time.perf_counter()
            gt, st = oracle.p2g_quadratic_threads(w.dim, w.n, w.frac_bits, sample, rng, threads)
            tt.append(time.perf_counter() - t)
            same = bool(np.array_equal(g1, gt) and s1.tolist() == st.tolist())
            del g1, gt
            if not same:
                raise SystemExit("bench.py: the threaded oracle's grid differs from the single-thread oracle's")
        dt1, dtt = float(np.median(t1)), float(np.median(tt))
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as fh:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
        except OSError:
            pass
        gpu_rate = binned / (p2g_ms * 1e-3)
        out["cpu_baseline"] = {"value": round(n_s / dtt, 1), "unit": "particles/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the oracle's P2G over the first {n_s} particles of {w.name} on {threads} "
                                         f"host threads (private int64 grids, integer-summed), median of {runs} runs "
                                         f"{dtt:.2f}s; grid bit-identical to the one-thread oracle's",
                               "single_core": {"value": round(n_s / dt1, 1), "unit": "particles/s", "cores": 1,
                                               "seconds": round(dt1, 3)},
                               "gpu_p2g_over_cpu": round(gpu_rate / (n_s / dtt), 1),
                               "host_cpu": cpu_model,
                               "host_cpus": os.cpu_count(), "host_cpus_usable": len(os.sched_getaffinity(0))}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
