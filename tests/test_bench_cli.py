"""bench.py's command-line contract on a machine without a GPU: more than one
GPU is refused with a message (this path runs on one GPU only), and the
counter-calibration and workload tables are well formed."""
import json
import os
import subprocess
import sys

import bench
from na3d_inputs import NORM_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line on refusal


def test_headline_workload_and_sizes():
    w = WORKLOADS[bench.HEADLINE]
    assert w.shape == (1, 16, 64, 96, 8, 64) and w.window == (3, 7, 7)
    assert w.flops == 4 * 98304 * 8 * 147 * 64
    assert w.bytes == 4 * 98304 * 8 * 64 * 2
    n = NORM_WORKLOADS["rms_block_norm"]
    assert n.bytes == 2 * 24576 * 4096 * 2 + 4096 * 2


def test_traffic_summaries_parse():
    # the committed counter summaries carry the fields bench.py reads
    for name, prof, src in (("decoder_tile", "na3d_fwd_roll_%s_traffic.md", bench.KERNEL_SOURCES),
                            ("rms_block_norm", "rms_norm_%s_traffic.md", bench.NORM_SOURCES)):
        text = open(os.path.join(ROOT, "profiles", prof % name)).read()
        assert "kernel_sources_sha256:" in text and "traffic_bytes_per_launch:" in text
        assert len(bench.sources_sha256(src)) == 64


def test_pages_grid_table():
    assert len(bench.PAGES_GRID) == 6
    for (T, H, W), ks, us in bench.PAGES_GRID:
        assert all(k <= n for k, n in zip(ks, (T, H, W))) and us > 0
    json.dumps([list(g) for g in bench.PAGES_GRID])


def test_provenance_helpers_run_without_a_gpu():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
    clocks = bench.gpu_clocks()
    assert "source" in clocks
    json.dumps(clocks)
