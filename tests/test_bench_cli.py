"""bench.py's command line on a machine without a GPU: more than one GPU is refused with a message (the
megakernel runs on one GPU), and every workload has a description and a default batch list."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_workload_descriptions():
    import bench
    from persistent_megakernel_mk_amd import synth

    assert bench.describe(synth.CONFIGS["c1"], 1).startswith("c1: hybrid 27B-class dense decode step")
    assert "verify step" in bench.describe(synth.CONFIGS["c2"], 1) and "8 rows" in bench.describe(synth.CONFIGS["c2"], 1)
    assert "384 experts top-8" in bench.describe(synth.CONFIGS["c3"], 8)
    assert "NVFP4" in bench.describe(synth.CONFIGS["c4"], 8) and "batch 8" in bench.describe(synth.CONFIGS["c4"], 8)
