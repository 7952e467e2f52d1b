"""Host-side logic of bench.py (no GPU): the refusal of more than one GPU, and
the lookup of measured HBM traffic, which must be dropped once the kernel's
sources differ from those the counters were taken on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_traffic_lookup_follows_the_kernel_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "kv_cache_compression_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "common.h").write_text("// common\n")
    (csrc / "select_topk.hip").write_text("// select, version 1\n")
    (csrc / "compact.hip").write_text("// compact\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest("select_topk")
    wl = "some-workload"
    table = ("| kernel | sources | fetch KiB | write KiB | algorithmic | measured | ratio |\n"
             "|---|---|---|---|---|---|---|\n"
             f"| select_topk | {digest} | 10 | 2 | 1000 | 1234 | 1.234 |\n"
             "| compact | 0000000000000000 | 1 | 1 | 1 | 1 | 1.0 |\n")
    (tmp_path / "profiles" / f"hbm-traffic_{wl}.md").write_text(table)
    assert bench.measured_traffic(wl, "select_topk") == 1234
    assert bench.measured_traffic(wl, "compact") is None          # other sources
    assert bench.measured_traffic("no-such-workload", "select_topk") is None
    (csrc / "select_topk.hip").write_text("// select, version 2\n")
    assert bench.source_digest("select_topk") != digest
    assert bench.measured_traffic(wl, "select_topk") is None      # sources changed since
