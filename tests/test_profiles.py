"""The committed rocprofv3 summaries stay tied to the code they measure.

The byte counters behind ``roofline.traffic`` (profiles/
score_kernel_<workload>_traffic.json) carry the hash of the score kernel's
sources they were taken on; bench.py reports them only while the hash
matches.  A change to those sources must come with new counter runs, so the
hash is checked here, on the CPU.  The kernel summaries must name every
kernel of the prune step, and bench.py refuses to report more than one GPU.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_traffic_counters_match_the_score_kernel_source():
    with open(bench.traffic_file("qwen3_32k")) as f:
        t = json.load(f)
    assert t["kernel_hash"] == bench.kernel_hash(), \
        "score kernel sources changed since the byte counters were taken: re-run the --pmc runs"
    assert t["workload"] == "qwen3_32k"
    # the request counters, turned into bytes by request size, read the plain
    # 1 GiB copy as 1 GiB read and 1 GiB written
    c = t["copy_requests"]
    assert abs(c["read_scale"] - 1.0) < 1e-3 and abs(c["write_scale"] - 1.0) < 1e-3
    # K read once (2,415,919,104 bytes), scores written once (37,748,736)
    k = t["kernels"]["score_kernel"]["requests"]
    assert abs(k["read_bytes_scaled"] / 2415919104 - 1.0) < 0.02
    assert abs(k["write_bytes_scaled"] / 37748736 - 1.0) < 0.02
    assert t["traffic_bytes_per_launch"] == k["read_bytes_scaled"] + k["write_bytes_scaled"]


def test_every_workload_has_fresh_counters():
    # each single-GPU workload whose score kernel was counted carries the
    # same source hash, and its score kernel reads each K row about once
    for w in ("qwen3_32k", "llama8b", "wide", "batched"):
        with open(bench.traffic_file(w)) as f:
            t = json.load(f)
        assert t["workload"] == w
        assert t["kernel_hash"] == bench.kernel_hash(), w
        k = t["kernels"]["score_kernel"]["requests"]
        _, k_read, _ = bench.workload_bytes(synth.workload(w))
        assert 0.99 < k["read_bytes_scaled"] / k_read < 1.03, w


def test_gqa_counters_match_the_gqa_kernel_source():
    # the GQA line's counters were taken on the current GQA kernel sources; the
    # kernel reads each K row about once and writes the raw scores and tile
    # statistics once, and the selection reads them back once
    kernel, sources = bench.score_kernel_of(4)
    with open(bench.traffic_file("qwen3_32k_gqa", kernel)) as f:
        t = json.load(f)
    assert t["workload"] == "qwen3_32k_gqa" and t["kernel"] == "gqa_mfma_kernel"
    assert t["kernel_hash"] == bench.kernel_hash(sources)
    sp = synth.workload("qwen3_32k_gqa")
    _, k_read, _ = bench.workload_bytes(sp)
    n = sp.lengths[0]
    inter = sp.heads * n * sp.group * 4 + sp.heads * ((n + 511) // 512) * sp.group * 32
    k = t["kernels"]["gqa_mfma_kernel"]["requests"]
    assert 0.99 < k["read_bytes_scaled"] / k_read < 1.03
    assert 0.99 < k["write_bytes_scaled"] / inter < 1.03
    sel = t["kernels"]["select_gqa_kernel"]["requests"]
    assert 0.99 < sel["read_bytes_scaled"] / inter < 1.03
    assert t["traffic_bytes_per_launch"] == k["read_bytes_scaled"] + k["write_bytes_scaled"]


STEP_KERNELS = {
    "qwen3_32k": ("score_kernel<128, true>", "select_reg_kernel<32, 1024, false>",
                  "compact_kernel<256, 1>"),
    "llama8b": ("score_kernel<128, true>", "select_reg_kernel<", "compact_kernel<256, 1>"),
    "wide": ("score_kernel<128, true>", "select_wide_kernel", "compact_kernel<256, 1>"),
    "batched": ("score_kernel<128, true>", "select_batch_kernel<32>", "select_batch_kernel<24>",
                "select_batch_kernel<16>", "select_batch_kernel<8>", "compact_batch_kernel<256>"),
    "qwen3_32k_gqa": ("gqa_prep_kernel<128, 4>", "gqa_mfma_kernel<128, 4>",
                      "select_gqa_kernel<32, 4>", "compact_kernel<256, 1>"),
    "shared_floor1024": ("select_reg_kernel<32, 1024, true>", "shared_pass_kernel",
                         "shared_write_kernel<32>", "order_kernel", "compact_kernel<256, 2>"),
}


def test_next_row_summaries_exist():
    for name, kernel in (("calib_stats_qwen3_kernel_stats.md", "calib_stats_kernel<128, true>"),
                         ("distance_curve_qwen3_gqa_kernel_stats.md", "distance_curve_kernel")):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
        assert "rocprofv3 --kernel-trace --stats" in text and kernel in text, name


def test_kernel_summaries_name_the_step_kernels():
    for w, kernels in STEP_KERNELS.items():
        path = os.path.join(ROOT, "profiles", "prune_step_%s_kernel_stats.md" % w)
        with open(path) as f:
            text = f.read()
        assert "rocprofv3 --kernel-trace --stats" in text, w
        for k in kernels:
            assert k in text, (w, k)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")
