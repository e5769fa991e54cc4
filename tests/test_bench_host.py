"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
ALU operation count per particle, and the traffic lookup from the committed
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
    import bench
    # per node: w*m*S, 3 sums for u, 3 momentum products, 4 roundings, 4 widenings, 3 float64 adds
    assert bench.alu_ops_per_node(3) * 27 == 486
    # 2D: 1 + 2 + 2 + 3 + 3 + 2.25 per node over 9 nodes
    assert bench.alu_ops_per_node(2) * 9 == pytest.approx(119.25)
    assert bench.VALU_PEAK_TOPS == pytest.approx(39.3216)


def test_traffic_lookup_is_none_when_the_summary_is_missing(tmp_path, monkeypatch):
    import bench
    # a copy of bench.py beside no profiles/ directory finds no summary
    d = tmp_path / "repo"
    (d / "material_point_particle_amd" / "csrc").mkdir(parents=True)
    for f in ("p2g.hip", "p2g_device.hpp", "common.hpp"):
        src = os.path.join(ROOT, "material_point_particle_amd", "csrc", f)
        (d / "material_point_particle_amd" / "csrc" / f).write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(d / "bench.py"))
    assert bench.measured_traffic() is None
