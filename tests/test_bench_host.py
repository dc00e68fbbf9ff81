"""Host-side checks of bench.py that need no GPU: the one-GPU contract, and that the committed
rocprofv3 counter summaries still belong to the kernel sources they were taken from (bench.py
reports `traffic` and `mfma_counters` as null otherwise)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus_requested"] == 2 and "one GPU" in msg["error"]


def test_traffic_summary_matches_the_gemv_sources():
    t = bench.kernel_traffic()
    assert t is not None, "profiles/gemv_decode70b_m1_traffic.json predates gemv.hip / bl_internal.h"
    # HBM bytes per launch within a few percent of the algorithmic bytes of a 70B pass launch
    # (weights + fp16 x + fp32 y, 17,148,149,760 B over 320 launches)
    assert 0.98 < t / (17148149760 / 320) < 1.10


def test_mfma_summary_matches_the_gemm_sources():
    s = bench.mfma_counters()
    assert s is not None, "profiles/gemm_prefill3b_m512_mfma.json predates tern_mfma.hip / bl_internal.h"
    for name, v in s.items():
        if isinstance(v, dict):
            assert 0.0 < v["mfma_util_pct"] <= 100.0, name
    assert 90.0 < s["calibration_mfma_i8_kernel_util_pct"] <= 100.0
