"""Host-side checks of bench.py's contract (no GPU): one-GPU only, and the
algorithmic work figures behind its roofline."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_of_the_rebuild_and_context_kernels():
    # one rebuild layer's gate/up: 2 * 768 * 2048 * 2 * 16384 FLOP; weights + x + h bytes
    f, b = bench.site_work("rebuild.glu", 231, [1229], rebuild_rows=768)
    assert f == 2.0 * 768 * 2048 * 2 * 16384 == 103079215104.0
    assert b == 2 * 16384 * 2048 * 2 + 768 * 2048 * 2 + 768 * 16384 * 2
    # by default a rebuild launch covers the call's batch of 4 entering entries
    f4, b4 = bench.site_work("rebuild.glu", 231, [1229])
    assert f4 == 4 * f and b4 == 2 * 16384 * 2048 * 2 + 4 * (768 * 2048 * 2 + 768 * 16384 * 2)
    f, b = bench.site_work("ctx.down", 231, [1229])
    assert f == 2.0 * 231 * 16384 * 2048
    assert b == 2048 * 16384 * 2 + 231 * 16384 * 2 + 231 * 2048 * 2
    assert bench.site_work("act.finish", 231, [1229]) is None


def test_stored_traffic_matches_only_current_sources():
    t, src = bench.stored_traffic("rebuild.glu")
    assert (t is None) == (src is None)
    assert bench.stored_traffic("no.such.kernel") == (None, None)
