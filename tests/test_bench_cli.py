"""bench.py's command line on the CPU: more than one GPU is refused before anything touches a
device, and the oracle baseline's bookkeeping (no GPU involved)."""
import os
import subprocess
import sys

import numpy as np

import oracle
import pa_inputs


def test_more_than_one_gpu_exits_with_a_message(root_dir):
    r = subprocess.run([sys.executable, os.path.join(root_dir, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_passes_over_the_rows_within_its_budget(root_dir):
    sys.path.insert(0, root_dir)
    import bench
    w = pa_inputs.make_workload(name="tiny", seq_lens=[5, 40, 17], block_size=16, seed=3)
    ref = oracle.paged_attention_workload(w)
    r = bench.cpu_baseline(w, ref, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1
    assert r["value"] > 0
    # compared against the oracle's own output: exactly zero difference
    assert r["max_abs_err_vs_gpu"] == 0.0
    # several passes over three short rows fit in 0.2 s
    assert "whole passes over the 3 rows" in r["sample"]
    n = int(r["sample"].split(" row evaluations")[0])
    assert n >= 3
    assert np.isfinite(r["kv_tokens_per_s"])
