"""Host-side checks of bench.py: the committed counter summaries it reads, and
its refusal of more than one GPU. No GPU needed."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_summary_parses():
    # a stored HBM traffic figure belongs to one workload and one kernel: a
    # kernel without a summary (or whose sources changed since) gets None
    t = bench.stored_traffic("verify_dcp8")
    assert t is None or t > 0
    t = bench.stored_traffic("long_context_dcp8", "persistent")
    assert t is None or t > 0
    assert bench.stored_traffic("verify_dcp8", "split") is None
    assert bench.stored_traffic("no_such_workload") is None


def test_mfma_summaries_parse_and_agree_with_instruction_count():
    for wl, route in (("verify_dcp8", "shards"), ("ragged_mixed", "persistent"),
                      ("long_context_dcp8", "persistent")):
        if not os.path.exists(bench.summary_path(wl, route, "mfma")):
            continue
        f = bench.stored_mfma_flops(wl, route)
        if f is None:              # summary taken before the kernel last changed
            continue
        # every v_mfma_f32_32x32x16_bf16 is 32768 flops: the executed count is a
        # whole number of instructions
        assert f > 0 and abs(f / 32768 - round(f / 32768)) < 1e-3 * (f / 32768)
    assert bench.stored_mfma_flops("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
