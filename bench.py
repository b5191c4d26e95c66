"""Benchmark of one TriAttention prune step (score every cached key, select the
top-B per KV head, compact K/V/positions in place) on one MI355X.

Default workload: the Qwen3-8B-shaped 32K reasoning cache (36 layers x 8 KV
heads x head_dim 128, 32768 cached keys per head, budget 4096, bf16), synthetic
and seeded.  A step is one whole prune pass over every head, with inputs
resident in HBM.  Between steps the cache is restored from a pristine device
copy (for caches above 64 GB, such as the 64-sequence batch, a copy of the
rows a step can overwrite) and a 512 MiB buffer is read to flush the 256 MB
last-level cache; both are outside the timed events.  The flush reads rather than writes: a written
flush buffer leaves up to 256 MB of dirty lines whose write-back then lands
inside the timed step (measured: ~12 us per step), while a read evicts the
restore's dirty lines before the first event.  Times come from HIP events
recorded on the stream the kernels run on: the timed steps carry one event
before the first launch and one after the last; the per-phase breakdown (and
the score kernel's duration for the roofline) comes from up to ten further
steps with events between the launches.

Prints one JSON line.  Extra modes:
  --pmc-steps N      a plain 1 GiB device copy, then N steps with no restores
                     (for rocprofv3 counter runs; see --summarize-pmc)
  --summarize-pmc D  turn rocprofv3 counter CSVs under D (runs of --pmc-steps N
                     on --workload W) into profiles/K_W_traffic.json (K the
                     score-phase kernel: score_kernel, or gqa_mfma_kernel for
                     GQA), which later runs report as roofline.traffic
  --shared-floor F   head-specific budgets: the KV heads of a layer share
                     budget * n_kv_heads slots, each keeping at least its F
                     best keys (shared select and counted compaction)
  --calib-stats N, --distance-curve N   time those calls instead
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6
METRIC = "cached keys scored+pruned/sec (G keys/s) and achieved HBM GB/s vs peak"
SCORE_KERNEL = "score_kernel"
GQA_SCORE_KERNEL = "gqa_mfma_kernel"
# each score kernel's sources (tri_internal.h holds only declarations shared
# by every kernel file, so it is not part of the hash)
KERNEL_SOURCES = ["rope_aware_eviction_amd/csrc/score.hip"]
GQA_KERNEL_SOURCES = ["rope_aware_eviction_amd/csrc/gqa.hip", "rope_aware_eviction_amd/csrc/gqa_stats.h"]


def score_kernel_of(group: int):
    """(name, sources) of the kernel of the score phase: the single-table
    kernel, or the GQA matrix-core kernel (G > 1, the workloads' bf16 K)."""
    return (SCORE_KERNEL, KERNEL_SOURCES) if group == 1 else (GQA_SCORE_KERNEL, GQA_KERNEL_SOURCES)


def traffic_file(workload: str, kernel: str = SCORE_KERNEL) -> str:
    """Committed byte-counter summary of a score kernel on one workload."""
    return os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, workload))


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload_bytes(spec):
    """Algorithmic bytes of one prune step and of its score kernel.

    pass:   per firing head N*row (read K) + 4*B*row (read and write the kept K
            and V rows) + 8*B (read and write the kept positions); the scores
            are an intermediate and are not counted
    k_read: per head N*row, the K rows the score kernel must read once (its
            algorithmic bytes)
    score_io: what the score phase writes besides: 4*N of fp32 scores; with
            G > 1 query heads per KV head instead the G raw scores per key,
            4*G*N (the selection reads them back and forms the score)
    """
    H, row, B, G = spec.heads, spec.row_bytes, spec.budget, spec.group
    p = sum(H * (n * row + 4 * B * row + 8 * B) for n in spec.lengths if n > B + spec.window)
    k = sum(H * n * row for n in spec.lengths)
    io = sum(H * (4 * G * n if G > 1 else 4 * n) for n in spec.lengths)
    return p, k, io


def describe(spec) -> str:
    ln = spec.lengths
    lens = "%d cached keys" % ln[0] if len(ln) == 1 else "%d sequences, %d..%d keys" % (len(ln), min(ln), max(ln))
    gqa = ", %d query heads per KV head" % spec.group if spec.group > 1 else ""
    return "%s: %d layers x %d KV heads x head_dim %d%s, %s, budget %d, %s" % (
        spec.name, spec.n_layers, spec.n_kv_heads, spec.head_dim, gqa, lens, spec.budget, spec.dtype)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cache, n_heads_sample: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same cache:
    full prune (score, select, gather) of n_heads_sample heads, one head per
    host thread on every core the process may use, then one head on one
    thread.  Heads are the first ones of a one-sequence cache, or spread over
    the sequences (and their lengths) of a batch."""
    import torch
    import oracle

    orc = oracle.load()
    sp, cal = cache.spec, cache.calib
    threads = min(len(os.sched_getaffinity(0)), 64)
    om = orc.omega(sp.head_dim, sp.rope_theta)
    G = sp.group
    if sp.n_seq == 1:
        picks = [(0,) + divmod(hi, sp.n_kv_heads) for hi in range(n_heads_sample)]
    else:
        step = max(1, sp.n_seq // n_heads_sample)
        picks = [(s, (7 * s) % sp.n_layers, s % sp.n_kv_heads)
                 for s in range(0, sp.n_seq, step)][:n_heads_sample]

    def job(s, l, h):
        n = cache.lens[s]
        q = slice(h * G, (h + 1) * G) if G > 1 else h
        return dict(K=cache.k[s][l, h, :n].float().cpu().numpy(),
                    V=cache.v[s][l, h, :n].cpu().view(torch.int16).numpy(),
                    pos=cache.pos[s][l, h, :n].cpu().numpy(), p_now=cache.p_now[s], om=om,
                    offsets=cal.offsets, qc_re=cal.qc_re[l, q], qc_im=cal.qc_im[l, q],
                    q_mean_norm=cal.q_mean_norm[l, q], q_mrl=cal.q_mrl[l, q],
                    budget=sp.budget, window=sp.window)

    jobs = [job(*x) for x in picks]
    t0 = time.perf_counter()
    orc.prune_heads_parallel(jobs, threads)
    dt = time.perf_counter() - t0
    keys = sum(cache.lens[s] for s, _, _ in picks)
    t1 = time.perf_counter()
    orc.prune_heads_parallel(jobs[:1], 1)
    dt1 = time.perf_counter() - t1
    keys1 = cache.lens[picks[0][0]]
    return {"value": keys / dt / 1e9, "unit": "G keys/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "%d of %d heads, %d keys (full score+select+gather per head), %d threads "
                      "taking one head at a time, %.1f s wall"
                      % (len(picks), sp.heads * sp.n_seq, keys, threads, dt),
            "single_thread": {"value": keys1 / dt1 / 1e9, "unit": "G keys/s", "cores": 1,
                              "sample": "1 head, %d keys, %.2f s" % (keys1, dt1)}}


def cpu_baseline_shared(cache, n_layers_sample: int, floor: int):
    """The oracle's shared-budget prune (score every head of a layer, select
    over the layer, gather) on the first n_layers_sample layers."""
    import numpy as np
    import oracle

    orc = oracle.load()
    sp, cal = cache.spec, cache.calib
    threads = min(len(os.sched_getaffinity(0)), 64)
    om = orc.omega(sp.head_dim, sp.rope_theta)
    n, G = cache.lens[0], sp.group
    layers = []
    for l in range(n_layers_sample):
        heads = []
        for h in range(sp.n_kv_heads):
            q = slice(h * G, (h + 1) * G) if G > 1 else h
            heads.append(dict(
                K=cache.k[0][l, h, :n].float().cpu().numpy(),
                V=cache.v[0][l, h, :n].cpu().view(__import__("torch").int16).numpy(),
                pos=cache.pos[0][l, h, :n].cpu().numpy(), p_now=cache.p_now[0], om=om,
                offsets=cal.offsets, qc_re=cal.qc_re[l, q], qc_im=cal.qc_im[l, q],
                q_mean_norm=cal.q_mean_norm[l, q], q_mrl=cal.q_mrl[l, q]))
        layers.append(heads)
    t0 = time.perf_counter()
    for heads in layers:
        orc.prune_layer_shared(heads, sp.budget * sp.n_kv_heads, floor, sp.window,
                               threads=min(threads, len(heads)))
    dt = time.perf_counter() - t0
    keys = n_layers_sample * sp.n_kv_heads * n
    return {"value": keys / dt / 1e9, "unit": "G keys/s", "cores": min(threads, sp.n_kv_heads),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "%d of %d layers x %d KV heads x %d keys (score, shared select, gather), "
                      "%.1f s wall" % (n_layers_sample, sp.n_layers, sp.n_kv_heads, n, dt)}


def load_traffic(spec):
    """roofline.traffic from the committed counter summary of this workload, or
    None when absent or taken on a different score kernel source."""
    kernel, sources = score_kernel_of(spec.group)
    try:
        with open(traffic_file(spec.name, kernel)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash(sources) or t.get("workload") != spec.name:
        return None
    return t.get("traffic_bytes_per_launch")


# kernel classes the counter summaries report (the first name a kernel's
# full name contains decides its class)
PMC_KERNELS = ("gqa_score_kernel", "gqa_prep_kernel", "gqa_mfma_kernel", "gqa_norm_kernel",
               SCORE_KERNEL, "select_batch_kernel", "select_reg_kernel", "select_gqa_kernel",
               "select_kernel", "compact_batch_kernel", "compact_kernel", "copyBuffer")
REQ_COUNTERS = ("TCC_EA0_RDREQ", "TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B",
                "TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B")


def summarize_pmc(directory: str, workload: str, steps: int):
    """Reads rocprofv3 --pmc counter_collection CSVs of `bench.py --pmc-steps
    steps` runs and writes the traffic summary of the score phase (and of the
    step's other kernels) on one workload, per prune step.

    Two sets of runs are read.  The memory-side request counters of the L2
    by request size (TCC_EA0_RDREQ_32B / _64B / _128B; TCC_EA0_WRREQ with
    TCC_EA0_WRREQ_64B, the rest of the write requests being 32 bytes) give
    bytes directly; FETCH_SIZE and WRITE_SIZE (derived KiB) are kept beside
    them.  Each is checked against the plain 1 GiB device copy of the same
    run and scaled by it.  traffic_bytes_per_launch (per step: the score
    phase is one launch per sequence) is the request-counter figure."""
    import numpy as np

    def values(counter):
        """counter -> {kernel class: [per-dispatch values]}"""
        out = {}
        for p in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    name = r.get("Counter_Name", "")
                    if name.endswith("_sum"):
                        name = name[:-4]
                    if name != counter:
                        continue
                    kname = r.get("Kernel_Name", "")
                    for k in PMC_KERNELS:
                        if k in kname:
                            out.setdefault(k, []).append(float(r["Counter_Value"]))
                            break
        return out

    vals = {c: values(c) for c in ("FETCH_SIZE", "WRITE_SIZE") + REQ_COUNTERS}

    def per_step(counter, k):
        v = vals[counter].get(k)
        return sum(v) / steps if v else None

    def copy_val(counter):
        v = vals[counter].get("copyBuffer")
        return max(v) if v else None     # the 1 GiB copy is the run's largest copy

    def req_bytes(get):
        r32, r64, r128 = (get("TCC_EA0_RDREQ_%s" % x) for x in ("32B", "64B", "128B"))
        wr, w64 = get("TCC_EA0_WRREQ"), get("TCC_EA0_WRREQ_64B")
        if None in (r32, r64, r128, wr, w64):
            return None
        return {"rdreq": get("TCC_EA0_RDREQ"), "rdreq_32b": r32, "rdreq_64b": r64, "rdreq_128b": r128,
                "wrreq": wr, "wrreq_64b": w64, "read_bytes": 32 * r32 + 64 * r64 + 128 * r128,
                "write_bytes": 64 * w64 + 32 * (wr - w64)}

    import synth
    kernel, sources = score_kernel_of(synth.workload(workload).group)
    copy_bytes = float(1 << 30)
    out = {"workload": workload, "kernel": kernel, "kernel_hash": kernel_hash(sources),
           "steps": steps, "unit": "bytes per prune step (all launches of the kernel class)"}
    cr = req_bytes(copy_val)
    if cr:
        out["copy_requests"] = dict(cr, read_scale=copy_bytes / cr["read_bytes"],
                                    write_scale=copy_bytes / cr["write_bytes"])
    cf, cw = copy_val("FETCH_SIZE"), copy_val("WRITE_SIZE")
    if cf and cw:
        out["copy_derived"] = {"fetch_kib": cf, "write_kib": cw, "fetch_scale": copy_bytes / (cf * 1024.0),
                               "write_scale": copy_bytes / (cw * 1024.0)}
    per = {}
    for k in PMC_KERNELS[:-1]:
        entry = {}
        b = req_bytes(lambda c: per_step(c, k))
        if b and cr:
            b["read_bytes_scaled"] = b["read_bytes"] * out["copy_requests"]["read_scale"]
            b["write_bytes_scaled"] = b["write_bytes"] * out["copy_requests"]["write_scale"]
            entry["requests"] = b
        f, w = per_step("FETCH_SIZE", k), per_step("WRITE_SIZE", k)
        if f is not None and w is not None and "copy_derived" in out:
            entry["derived"] = {"fetch_kib": f, "write_kib": w,
                                "fetch_bytes_scaled": f * 1024.0 * out["copy_derived"]["fetch_scale"],
                                "write_bytes_scaled": w * 1024.0 * out["copy_derived"]["write_scale"]}
        if entry:
            entry["dispatches_per_step"] = len(vals["TCC_EA0_RDREQ_128B"].get(k) or
                                               vals["FETCH_SIZE"].get(k) or []) / steps
            per[k] = entry
    out["kernels"] = per
    sk = per.get(kernel, {})
    if "requests" in sk:
        out["traffic_bytes_per_launch"] = sk["requests"]["read_bytes_scaled"] + sk["requests"]["write_bytes_scaled"]
        out["traffic_from"] = "TCC_EA0 read and write requests by size, scaled by the 1 GiB copy"
    elif "derived" in sk:
        out["traffic_bytes_per_launch"] = sk["derived"]["fetch_bytes_scaled"] + sk["derived"]["write_bytes_scaled"]
        out["traffic_from"] = "FETCH_SIZE + WRITE_SIZE, scaled by the 1 GiB copy"
    path = traffic_file(workload, kernel)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def bench_calib_stats(args, torch, synth, tri, dev):
    """One JSON line for tri_calibrate_stats on Qwen3-8B-shaped query samples:
    36 layers x 32 query heads = 1152 heads, head_dim 128, bf16."""
    H, d, n = 36 * 32, 128, args.calib_stats
    print("bench: generating %d query samples of %d heads" % (n, H), file=sys.stderr, flush=True)
    q, _, _ = synth.query_samples(H, d, n, seed=args.seed, dtype="bf16", device=dev)
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        tri.tri_calibrate_stats(q)
    times = []
    for _ in range(args.steps):
        flush.sum(dtype=torch.int64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tri.tri_calibrate_stats(q, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sum(times) / len(times)
    nbytes = q.numel() * q.element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "calibration statistics from pre-RoPE query samples (samples per second)",
        "value": n / (ms * 1e-3), "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B query heads: 36 layers x 32 heads x head_dim 128",
                   "samples": n, "heads": H, "head_dim": d},
        "roofline": {"bound": "hbm", "kernel": "calib_stats_kernel", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "alg_bytes_per_launch": nbytes, "launch_ms": ms}}), flush=True)


def bench_distance_curve(args, torch, synth, tri, dev):
    """One JSON line for tri_distance_curve: 1152 query heads of the qwen3_32k_gqa
    calibration, N_DELTA distances 0..N_DELTA-1 (fp64; bound by fp64 sincos)."""
    spec = synth.workload("qwen3_32k_gqa")
    cal = synth._model(spec, args.seed)[2]
    ctx = tri.tri_calibrate_load(spec.n_layers, spec.n_kv_heads, spec.head_dim, cal.qc_re, cal.qc_im,
                                 cal.q_mean_norm, cal.q_mrl, cal.offsets, rope_theta=cal.rope_theta,
                                 device=0, n_q_heads=spec.n_q_heads)
    h = spec.head_dim // 2
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    kc_re = torch.randn((spec.heads, h), dtype=torch.float64, device=dev, generator=g)
    kc_im = torch.randn((spec.heads, h), dtype=torch.float64, device=dev, generator=g)
    deltas = torch.arange(args.distance_curve, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        tri.tri_distance_curve(ctx, kc_re, kc_im, deltas)
    times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tri.tri_distance_curve(ctx, kc_re, kc_im, deltas, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sum(times) / len(times)
    entries = spec.heads * spec.group * args.distance_curve
    terms = entries * h
    print(json.dumps({
        "metric": "distance-preference curve entries per second",
        "value": entries / (ms * 1e-3), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "qwen3_32k_gqa query heads: 36 x 8 x 4, head_dim 128",
                   "query_heads": spec.heads * spec.group, "deltas": args.distance_curve},
        # fp64 vector arithmetic: each (entry, band) term is two multiply-adds
        # (4 flops) against the accumulator; the phasors (one sincos per
        # distance, band and 64-head tile) are not counted.  Peak: MI355X fp64
        # vector, 78.6 TFLOP/s (256 CUs x 2.4 GHz x 128 flops per clock).
        "roofline": {"bound": "alu", "kernel": "distance_curve_kernel",
                     "achieved": 4 * terms / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                     "peak": FP64_PEAK_TFLOPS, "frac": 4 * terms / (ms * 1e-3) / 1e12 / FP64_PEAK_TFLOPS,
                     "traffic": None, "band_terms_per_s": terms / (ms * 1e-3)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="heads of the cache the oracle baseline prunes (0 = skip)")
    ap.add_argument("--pmc-steps", type=int, default=0)
    ap.add_argument("--summarize-pmc", default=None, metavar="DIR",
                    help="write profiles/<score kernel>_<workload>_traffic.json from the counter "
                         "CSVs under DIR (with --workload)")
    ap.add_argument("--calib-stats", type=int, default=0, metavar="N_SAMPLES",
                    help="measure tri_calibrate_stats instead: N_SAMPLES pre-RoPE query samples of "
                         "the Qwen3-8B query heads (36 layers x 32 heads x head_dim 128, bf16)")
    ap.add_argument("--shared-floor", type=int, default=-1, metavar="F",
                    help="head-specific budgets with a per-head floor of F keys (default: off)")
    ap.add_argument("--distance-curve", type=int, default=0, metavar="N_DELTA",
                    help="measure tri_distance_curve instead: the curves of the 1152 Qwen3-8B "
                         "query heads (36 layers x 8 KV heads x 4) at N_DELTA distances")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, max(1, args.pmc_steps))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the pass is independent per (sequence, layer, "
              "KV head) and needs no collectives, so N GPUs each run this on their own share; "
              "run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import rope_aware_eviction_amd as tri

    tri.library()                       # fails loudly when the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.calib_stats:
        bench_calib_stats(args, torch, synth, tri, dev)
        return
    if args.distance_curve:
        bench_distance_curve(args, torch, synth, tri, dev)
        return
    spec = synth.workload(args.workload, seed=args.seed)
    print("bench: generating %s" % describe(spec), file=sys.stderr, flush=True)
    cache = synth.make_cache(spec, dev, seed=args.seed)
    cal = cache.calib
    ctx = tri.tri_calibrate_load(spec.n_layers, spec.n_kv_heads, spec.head_dim, cal.qc_re, cal.qc_im,
                                 cal.q_mean_norm, cal.q_mrl, cal.offsets, rope_theta=cal.rope_theta,
                                 device=0, n_q_heads=spec.n_q_heads)
    H, B, W = spec.heads, spec.budget, spec.window
    total = sum(H * n for n in cache.lens)
    scores = torch.empty(total, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    shared = args.shared_floor >= 0
    F = args.shared_floor
    if shared:
        # head-specific budgets: kept lists of up to budget * n_kv_heads per head,
        # per-head counts and lengths
        kstride = B * spec.n_kv_heads
        kept = torch.empty(spec.n_seq * H * kstride, dtype=torch.int32, device=dev)
        counts = torch.empty(spec.n_seq * H, dtype=torch.int32, device=dev)
        head_len = [torch.full((spec.n_layers, spec.n_kv_heads), n, dtype=torch.int32, device=dev)
                    for n in cache.lens]
        sel_ws = torch.empty(tri.select_shared_workspace_bytes(ctx, spec.n_seq), dtype=torch.uint8,
                             device=dev)
        cmp_ws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device=dev)
    else:
        kept = torch.empty(spec.n_seq * H * B, dtype=torch.int32, device=dev)

    def seqs():
        return [tri.Seq(cache.k[s], cache.v[s], cache.pos[s], cache.lens[s], cache.p_now[s],
                        head_len[s] if shared else None)
                for s in range(spec.n_seq)]

    # GQA contexts score through a workspace (G raw scores per key)
    ws_bytes = tri.score_workspace_bytes(ctx, seqs())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    # GQA with uniform budgets: the selection forms the aggregated score from
    # the raw per-query-head scores in the workspace (no score array written)
    gqa_ws = spec.group > 1 and not shared
    long_heads = max(cache.lens) > 32768

    def score(s):
        tri.tri_score(ctx, s, None if gqa_ws else scores, stream, ws)

    def select(s):
        if shared:
            tri.tri_select_shared(ctx, s, scores, B, F, W, kept, counts, sel_ws, stream)
        elif gqa_ws:
            tri.tri_select_topb_ws(ctx, s, ws, B, W, kept, stream, scores if long_heads else None)
        else:
            tri.tri_select_topb(ctx, s, scores, B, W, kept, stream)

    def compact(s):
        if shared:
            tri.tri_compact_kv_counts(ctx, s, kept, kstride, counts, cmp_ws, stream)
        else:
            tri.tri_compact_kv(ctx, s, kept, B, W, stream)

    def step(s):
        score(s)
        select(s)
        compact(s)

    if args.pmc_steps:
        # counter runs: one plain 1 GiB device copy (the scale for the byte
        # counters) and a few steps; no restores, so that copy is the only
        # large copy in the run.  Later steps score the compacted cache,
        # which moves the same bytes through the score kernel.
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        for _ in range(args.pmc_steps):
            step(seqs())
        torch.cuda.synchronize()
        print("pmc steps done", file=sys.stderr, flush=True)
        return

    # Restores: a full pristine copy of K, V and positions, or, when that
    # would not fit beside the cache (the 64-sequence batch holds ~155 GB),
    # a copy of the rows a step can overwrite: compaction writes only rows
    # below the kept count (budget, or budget x KV heads when the heads of a
    # layer share it), so restoring those rows restores the cache.
    kv_bytes = sum(2 * k.numel() * k.element_size() for k in cache.k)
    partial = kv_bytes > (64 << 30)
    rows = B * spec.n_kv_heads if shared else B
    if partial:
        pristine = [(k[:, :, :rows].clone(), v[:, :, :rows].clone(), p[:, :, :rows].clone())
                    for k, v, p in zip(cache.k, cache.v, cache.pos)]
    else:
        pristine = [(k.clone(), v.clone(), p.clone()) for k, v, p in zip(cache.k, cache.v, cache.pos)]
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    def restore():
        for (k0, v0, p0), k, v, p in zip(pristine, cache.k, cache.v, cache.pos):
            r = k0.shape[2]
            k[:, :, :r].copy_(k0)
            v[:, :, :r].copy_(v0)
            p[:, :, :r].copy_(p0)
        if shared:
            for hl, n in zip(head_len, cache.lens):
                hl.fill_(n)
        flush.sum(dtype=torch.int64)      # reads 512 MiB: evicts the cache, leaves it clean

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        restore()
        step(seqs())
    torch.cuda.synchronize()
    print("bench: warmup done; timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        restore()                        # untimed: outside the events
        s = seqs()
        e = ev[i]
        e[0].record(stream)
        step(s)
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_step = [e[0].elapsed_time(e[1]) for e in ev]

    # Phase breakdown from separate steps: an event between two launches
    # costs a few microseconds, so the timed steps above carry none.
    n_phase = max(1, min(args.steps, 10))
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_phase)]
    for i in range(n_phase):
        restore()
        s = seqs()
        e = pev[i]
        e[0].record(stream)
        score(s)
        e[1].record(stream)
        select(s)
        e[2].record(stream)
        compact(s)
        e[3].record(stream)
    torch.cuda.synchronize()
    t_score = [e[0].elapsed_time(e[1]) for e in pev]
    t_select = [e[1].elapsed_time(e[2]) for e in pev]
    t_compact = [e[2].elapsed_time(e[3]) for e in pev]

    # The score kernel's duration for the roofline is the score interval of
    # these steps: it holds one dispatch gap (~5 us) that the profiler's
    # per-dispatch durations do not.  Timing score phases back to back instead
    # hides the gap but not the write-back of the previous phase's scores
    # (151 MB with four query heads per KV head), so each phase here starts
    # after a restore and a flush, as in a step.
    t_score_run = sum(t_score) / len(t_score)

    mean = lambda x: sum(x) / len(x)
    ms = mean(t_step)
    keys = spec.keys
    bytes_pass, bytes_k, bytes_score_io = workload_bytes(spec)
    score_gbs = bytes_k / (t_score_run * 1e-3) / 1e9
    pass_gbs = bytes_pass / (ms * 1e-3) / 1e9

    if shared:
        # every layer fired: the counts of a layer sum to its shared total
        c = counts.view(-1, spec.n_kv_heads)
        assert bool((c.sum(1) == B * spec.n_kv_heads).all()), "a layer did not keep its total"

    out = {
        "metric": METRIC,
        "value": keys / (ms * 1e-3) / 1e9,
        "unit": "G keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": describe(spec), "layers": spec.n_layers, "kv_heads": spec.n_kv_heads,
                   "head_dim": spec.head_dim, "cached_keys": list(spec.lengths)[:1] if spec.n_seq == 1 else "ragged",
                   "budget": B, "window": W, "storage": spec.dtype, "offsets": len(spec.offsets),
                   "budgets": ("shared per layer (budget x %d KV heads), floor %d per head"
                               % (spec.n_kv_heads, F)) if shared else "uniform per head"},
        "roofline": {"bound": "hbm", "kernel": SCORE_KERNEL if spec.group == 1 else
                     "GQA score phase (gqa_prep_kernel, gqa_mfma_kernel; f32 K: gqa_score_kernel); "
                     "the selection forms the statistics and the aggregated score",
                     "achieved": score_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": score_gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic(spec),
                     # K rows read once: the score phase's algorithmic bytes
                     "alg_bytes_per_launch": bytes_k,
                     # not algorithmic: fp32 scores written (and GQA raw scores written and read)
                     "intermediate_bytes_per_launch": bytes_score_io,
                     # score-kernel launches per step (one per sequence) and
                     # the score phase's event-timed duration
                     "launches": spec.n_seq, "launch_ms": t_score_run,
                     "timed_phases": n_phase},
        "pass": {"alg_bytes": bytes_pass, "achieved_gbs": pass_gbs, "frac": pass_gbs / HBM_PEAK_GBS,
                 # with the scores written by the score phase and read back by
                 # the selection (not algorithmic: an intermediate)
                 "bytes_with_scores": bytes_pass + 2 * bytes_score_io,
                 "phase_ms": {"score": mean(t_score), "select": mean(t_select),
                              "compact": mean(t_compact)},
                 "step_ms_min": min(t_step), "step_ms_max": max(t_step),
                 "step_ms_median": sorted(t_step)[len(t_step) // 2]},
        "wall_s_timed_loop_incl_restores": wall,
        "cpu_baseline": None,
    }
    if args.cpu_heads > 0 and (spec.n_seq == 1 or not shared):
        restore()
        torch.cuda.synchronize()
        print("bench: oracle baseline on %d heads" % args.cpu_heads, file=sys.stderr, flush=True)
        if shared:
            out["cpu_baseline"] = cpu_baseline_shared(
                cache, max(1, min(args.cpu_heads // spec.n_kv_heads, spec.n_layers)), F)
        else:
            out["cpu_baseline"] = cpu_baseline(cache, min(args.cpu_heads, spec.heads))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
