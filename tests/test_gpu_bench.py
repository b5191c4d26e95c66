"""The benchmark's JSON contract, on small workloads (in-process): one line with
the metric, the throughput, the roofline of the dominant kernel and the CPU
baseline, for the uniform, head-specific-budget and GQA modes."""
import contextlib
import io
import json
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def run_bench(*argv):
    import bench
    out = io.StringIO()
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        with contextlib.redirect_stdout(out):
            bench.main()
    finally:
        sys.argv = old
    torch.cuda.synchronize()
    lines = [l for l in out.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


@pytest.mark.parametrize("argv", [
    ("--workload", "toy", "--steps", "3", "--warmup", "1", "--cpu-heads", "2"),
    ("--workload", "gqa_toy", "--steps", "3", "--warmup", "1", "--cpu-heads", "2"),
    ("--workload", "toy", "--steps", "3", "--warmup", "1", "--cpu-heads", "2",
     "--shared-floor", "16"),
])
def test_bench_prints_one_contract_line(argv):
    d = run_bench(*argv)
    assert KEYS <= set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"].split(":")[0] in ("toy", "gqa_toy")
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
