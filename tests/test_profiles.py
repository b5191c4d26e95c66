"""The committed rocprofv3 summaries stay tied to the code they measure.

The byte counters behind ``roofline.traffic`` (profiles/
score_kernel_qwen3_32k_traffic.json) carry the hash of the score kernel's
sources they were taken on; bench.py reports them only while the hash
matches.  A change to those sources must come with new counter runs, so the
hash is checked here, on the CPU.  The kernel summaries must name every
kernel of the prune step.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_counters_match_the_score_kernel_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["kernel_hash"] == bench.kernel_hash(), \
        "score kernel sources changed since the byte counters were taken: re-run the two --pmc runs"
    assert t["workload"] == "qwen3_32k"
    # K read once, scores written once: within 2% of the algorithmic bytes
    alg = 9437184 * 260
    assert abs(t["traffic_bytes_per_launch"] / alg - 1.0) < 0.02


def test_kernel_summaries_name_the_step_kernels():
    with open(os.path.join(ROOT, "profiles", "prune_step_qwen3_32k_kernel_stats.md")) as f:
        text = f.read()
    for k in ("score_kernel<128, true>", "select_reg_kernel<32, 1024, false>", "compact_kernel<256, 1>"):
        assert k in text, k
    with open(os.path.join(ROOT, "profiles", "shared_prune_step_qwen3_32k_kernel_stats.md")) as f:
        text = f.read()
    for k in ("select_reg_kernel<32, 1024, true>", "shared_pass_kernel", "shared_write_kernel<32>",
              "order_kernel", "compact_kernel<256, 2>"):
        assert k in text, k
