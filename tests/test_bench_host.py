"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
ALU operation count per particle by instruction class, the algorithmic byte
count, the stage statistics, and the profile lookup from the committed
counter summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_alu_operations_per_particle():
    import itertools

    import bench
    # count the distinct subexpressions of the fixed-order transfer by enumerating them
    for dim in (2, 3):
        offs = range(3)
        prefixes = {t for k in range(1, dim + 1) for t in itertools.product(offs, repeat=k)}
        nodes = list(itertools.product(offs, repeat=dim))
        weights = 18 * dim                                    # per-axis stencil setup
        wms = 1 + len(prefixes)                               # m*S, then ((m S wx) wy) wz prefixes
        u_products = {(e, a, o) for e in range(dim) for a in range(dim) for o in offs}   # C_ea * r_a[o]
        u_sums = {(e, t) for e in range(dim) for t in prefixes}
        momentum = dim * len(nodes)
        fast, slow = bench.alu_ops_per_particle(dim)
        assert fast == weights + wms + len(u_products) + len(u_sums) + momentum
        per_value = 1 + 1 + 0.75                              # round, widen, 3/4 of a float64 add
        assert slow == pytest.approx(2 * dim + per_value * (1 + dim) * len(nodes))
    assert bench.alu_ops_per_particle(3) == (319, pytest.approx(303))
    # the slow class issues one 64-lane instruction per SIMD every 4 cycles
    assert bench.SLOW_PEAK_TOPS == pytest.approx(39.3216)


def test_algorithmic_bytes_and_stage_stats():
    import numpy as np

    import bench
    # 3D: 64 B of state (x, v, C, m) + a 4-byte index entry per particle, 32 B per touched node
    assert bench.p2g_algorithmic_bytes(3, 10, 7) == 10 * 68 + 7 * 32
    assert bench.p2g_algorithmic_bytes(2, 10, 7) == 10 * 40 + 7 * 24     # 2D: 36 B of state + 4
    st = bench.stage_stats(np.arange(1, 11, dtype=float))
    assert st["median"] == 5.5 and st["mean"] == 5.5 and st["p10"] == pytest.approx(1.9)
    assert st["p90"] == pytest.approx(9.1)


def test_profile_lookup_is_none_when_the_summary_is_missing(tmp_path, monkeypatch):
    import bench
    # a copy of bench.py beside no profiles/ directory finds no summary
    d = tmp_path / "repo"
    (d / "material_point_particle_amd" / "csrc").mkdir(parents=True)
    for f in ("p2g.hip", "p2g_device.hpp", "common.hpp"):
        src = os.path.join(ROOT, "material_point_particle_amd", "csrc", f)
        (d / "material_point_particle_amd" / "csrc" / f).write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(d / "bench.py"))
    assert bench.profile_record() is None
