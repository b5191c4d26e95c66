"""The GQA step (score into the workspace, select from it, compact) and the
head-specific-budget step (score, shared select, counted compaction) launch
kernels only, with every scratch buffer a caller-owned workspace, so a
caller can capture them in a HIP graph.  Each graph is replayed three times,
the cache (and head lengths) restored eagerly and synchronized between
replays, and every replay equals the eager step bit for bit."""
import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri
from test_gpu_parity import bits, say

pytestmark = pytest.mark.gpu


def _ctx(cache):
    sp, cal = cache.spec, cache.calib
    return tri.tri_calibrate_load(sp.n_layers, sp.n_kv_heads, sp.head_dim, cal.qc_re, cal.qc_im,
                                  cal.q_mean_norm, cal.q_mrl, cal.offsets,
                                  rope_theta=cal.rope_theta, device=0, n_q_heads=sp.n_q_heads)


def _replay_equals_eager(cache, restore, step, outs):
    restore()
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs()]
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(bits(a) if a.is_floating_point() else a,
                               bits(b) if b.is_floating_point() else b), "replay %d" % r


def test_gqa_step_replays_from_a_hip_graph():
    sp = synth.workload("gqa_small").replace(lengths=(4001, 2600), budget=900)
    cache = synth.make_cache(sp, "cuda", seed=50)
    ctx = _ctx(cache)
    pristine = [(k.clone(), v.clone(), p.clone()) for k, v, p in zip(cache.k, cache.v, cache.pos)]

    def seqs():
        return [tri.Seq(cache.k[s], cache.v[s], cache.pos[s], cache.lens[s], cache.p_now[s])
                for s in range(sp.n_seq)]

    ws = torch.empty(tri.score_workspace_bytes(ctx, seqs()), dtype=torch.uint8, device="cuda")
    kept = torch.full((sp.n_seq * sp.heads * sp.budget,), -1, dtype=torch.int32, device="cuda")

    def restore():
        for (k0, v0, p0), k, v, p in zip(pristine, cache.k, cache.v, cache.pos):
            k.copy_(k0)
            v.copy_(v0)
            p.copy_(p0)
        kept.fill_(-1)

    def step():
        tri.prune_step_gqa(ctx, seqs(), sp.budget, sp.window, kept, ws)

    _replay_equals_eager(cache, restore, step,
                         lambda: [kept] + [x for s in range(sp.n_seq)
                                           for x in (cache.k[s], cache.v[s], cache.pos[s])])
    say("  GQA step: three graph replays equal the eager step")


def test_shared_step_replays_from_a_hip_graph():
    sp = synth.workload("llama8b").replace(name="graph_shared", n_layers=2, lengths=(6000,),
                                           budget=500)
    L, H1, n = sp.n_layers, sp.n_kv_heads, sp.lengths[0]
    cache = synth.make_cache(sp, "cuda", seed=51)
    ctx = _ctx(cache)
    hl0 = torch.from_numpy(synth.head_lengths("ragged", L, H1, n, seed=3)).cuda()
    head_len = hl0.clone()
    K0, V0, P0 = cache.k[0].clone(), cache.v[0].clone(), cache.pos[0].clone()
    total = sp.budget * H1
    scores = torch.empty(L * H1 * n, device="cuda")
    kept = torch.full((L * H1 * total,), -1, dtype=torch.int32, device="cuda")
    counts = torch.empty((L * H1,), dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, 1), dtype=torch.uint8, device="cuda")
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")

    def restore():
        cache.k[0].copy_(K0)
        cache.v[0].copy_(V0)
        cache.pos[0].copy_(P0)
        head_len.copy_(hl0)
        kept.fill_(-1)
        counts.fill_(-7)

    def step():
        seq = tri.Seq(cache.k[0], cache.v[0], cache.pos[0], n, cache.p_now[0], head_len)
        tri.prune_step_shared(ctx, [seq], sp.budget, 64, sp.window, scores, kept, counts, ws, cws)

    _replay_equals_eager(cache, restore, step,
                         lambda: [kept, counts, head_len, cache.k[0], cache.v[0], cache.pos[0]])
    assert int((counts >= 0).sum()) > 0, "no layer fired"
    say("  shared-budget step: three graph replays equal the eager step")
