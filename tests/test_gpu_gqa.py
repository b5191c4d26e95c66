"""GPU parity of the GQA normalize-then-aggregate score (tri_score_ws)
against the fp64 oracle, called through the C ABI.

Source: dimensionstp.github.io TriAttention review, section 3-2 item 6, and
romaanj.github.io TriAttention review, section "Method".

Bar (derived from the arithmetic): the GPU's raw per-query-head scores carry
the single-head score error, at most e * M_{g,i} with e = 2e-3 and M the
oracle's per-key bound; the mean then moves by at most e * mean(M_g) and the
deviation by at most e * rms(M_g), so
    |z_gpu - z_ref| <= e * (M_{g,i} + mean(M_g) + |z_ref| * rms(M_g)) / sd_g,
and the max over the group inherits the largest of these.  Kept sets are
checked as in the single-head parity tests with that per-key tolerance:
keys clearly above the B-th aggregated score are kept, keys clearly below
are evicted, disagreements lie within 1/20 of the tolerance band of the
threshold.  GPU-internal properties (ascending kept lists of B keys that are
the top-B of the GPU's own scores, bit-exact compaction, run-to-run
determinism) are checked on every head.
"""
import sys

import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri
from test_gpu_parity import bits, check_topb_property, head_inputs, say, seqs_for

pytestmark = pytest.mark.gpu

TOL = 2e-3
TIGHT = TOL / 20


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.load()


def ctx_gqa(cache):
    sp, cal = cache.spec, cache.calib
    return tri.tri_calibrate_load(sp.n_layers, sp.n_kv_heads, sp.head_dim, cal.qc_re, cal.qc_im,
                                  cal.q_mean_norm, cal.q_mrl, cal.offsets,
                                  rope_theta=cal.rope_theta, device=0, n_q_heads=sp.n_q_heads)


def workspace_for(ctx, seqs):
    n = tri.score_workspace_bytes(ctx, seqs)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def oracle_gqa(orc, cache, s, l, h, K, P):
    """Aggregated score, per-key tolerance and the per-query-head pieces."""
    sp, cal = cache.spec, cache.calib
    G = sp.group
    om = orc.omega(sp.head_dim, sp.rope_theta)
    rows = slice(h * G, (h + 1) * G)
    args = (cal.qc_re[l, rows], cal.qc_im[l, rows], cal.q_mean_norm[l, rows], cal.q_mrl[l, rows])
    raw, z, score = orc.gqa_head(K, P, cache.p_now[s], om, cal.offsets, *args)
    tol = np.zeros(len(score))
    for g in range(G):
        M = orc.bound_head(K, om, cal.offsets, cal.qc_re[l, h * G + g], cal.qc_im[l, h * G + g],
                           cal.q_mean_norm[l, h * G + g], cal.q_mrl[l, h * G + g])
        fin = np.isfinite(raw[g])
        sd = raw[g][fin].std()
        if sd > 0:
            zg = np.where(np.isfinite(z[g]), np.abs(z[g]), 0.0)
            tg = TOL * (M + M[fin].mean() + zg * np.sqrt((M[fin] ** 2).mean())) / sd
            tol = np.maximum(tol, tg)
    return score, tol


def check_agg(s_gpu, s_ref, tol, what):
    assert np.array_equal(np.isnan(s_gpu), np.isnan(s_ref)), what + ": NaN pattern differs"
    m = ~np.isnan(s_ref)
    err = np.abs(s_gpu[m].astype(np.float64) - s_ref[m])
    ratio = err / np.maximum(tol[m], 1e-300)
    say("  %s: max |dz| = %.3g, max |dz|/tol = %.3g over %d keys" % (what, err.max(), ratio.max(), m.sum()))
    assert np.all(err <= tol[m]), what


def check_kept(orc, s_ref, tol, P, kept_gpu, B, window, what):
    n = len(s_ref)
    kept_ref = orc.select_head(s_ref, P, B, window)
    key = np.where(np.isnan(s_ref), -np.inf, s_ref)
    order = np.lexsort((P, -key))
    ti = order[B - 1]
    t, tt = key[ti], tol[ti]
    sel = np.zeros(n, bool)
    sel[kept_gpu] = True
    assert sel.sum() == B
    band = tol + tt
    assert sel[key > t + band].all(), what + ": a clearly kept key was evicted"
    assert not sel[key < t - band].any(), what + ": a clearly evicted key was kept"
    ref = np.zeros(n, bool)
    ref[kept_ref] = True
    dis = np.nonzero(ref != sel)[0]
    if len(dis):
        assert np.all(np.abs(key[dis] - t) <= (TIGHT / TOL) * band[dis]), what
    say("  %s: kept-set disagreements with the oracle: %d of %d" % (what, len(dis), B))


@pytest.mark.parametrize("name,heads,over", [
    ("gqa_toy", None, None), ("gqa_small", None, None), ("gqa_g7", 2, None), ("gqa_g8_d64", 2, None),
    # fp32 K at head_dim 128 (the vector-unit kernel), and a length that ends
    # inside a 16-row group and a 512-row tile (the matrix-core kernel's tails)
    ("gqa_small", 2, {"dtype": "f32", "name": "gqa_small_f32"}),
    ("gqa_small", None, {"lengths": (4001,), "name": "gqa_small_4001"}),
    ("gqa_g8_d64", None, {"lengths": (530,), "name": "gqa_g8_d64_530"})])
def test_gqa_scores_match_oracle(orc, name, heads, over):
    spec = synth.workload(name)
    if over:
        spec = spec.replace(**over)
    say("gqa scores", spec.name, "G =", spec.group)
    cache = synth.make_cache(spec, "cuda", seed=3)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    n = cache.lens[0]
    scores = torch.full((spec.heads * n,), float("nan"), device="cuda")
    tri.tri_score(ctx, seqs, scores, workspace=ws)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy().reshape(spec.n_layers, spec.n_kv_heads, n)
    pairs = [(l, h) for l in range(spec.n_layers) for h in range(spec.n_kv_heads)]
    if heads is not None:
        pairs = [pairs[0], pairs[-1]][:heads]
    for l, h in pairs:
        K, _, P = head_inputs(cache, 0, l, h)
        s_ref, tol = oracle_gqa(orc, cache, 0, l, h, K, P)
        check_agg(sg[l, h], s_ref, tol, "%s l%d h%d" % (spec.name, l, h))


@pytest.mark.parametrize("name,over", [
    ("gqa_small", {"lengths": (4001, 301), "name": "gqa_small_two"}),
    ("gqa_g7", {"lengths": (530,), "name": "gqa_g7_530"}),
    ("gqa_g8_d64", {"lengths": (530,), "name": "gqa_g8_d64_530"}),
    ("gqa_small", {"lengths": (777,), "dtype": "f32", "name": "gqa_small_f32_777"})])
def test_gqa_scores_do_not_depend_on_the_workspace_address(name, over):
    """A head's score tiles follow from its length alone, so the per-tile
    statistics are summed in the same groups wherever the workspace lies:
    scores from a workspace at several 16-byte offsets are bit-identical."""
    spec = synth.workload(name).replace(**over)
    say("gqa workspace address", spec.name, "G =", spec.group, spec.lengths)
    cache = synth.make_cache(spec, "cuda", seed=5)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    need = tri.score_workspace_bytes(ctx, seqs)
    big = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    total = sum(spec.heads * n for n in cache.lens)
    ref = None
    for off in (0, 16, 80):
        scores = torch.full((total,), float("nan"), device="cuda")
        tri.tri_score(ctx, seqs, scores, workspace=big[off:off + need])
        torch.cuda.synchronize()
        got = scores.view(torch.int32).clone()
        if ref is None:
            ref = got
        else:
            assert torch.equal(got, ref), "workspace offset %d" % off


def test_gqa_needs_its_workspace():
    spec = synth.workload("gqa_toy")
    cache = synth.make_cache(spec, "cuda", seed=4)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    scores = torch.empty(spec.heads * cache.lens[0], device="cuda")
    with pytest.raises(tri.TriError) as e:
        tri.tri_score(ctx, seqs, scores)
    assert e.value.status == tri.TRI_E_INVAL
    small = torch.empty(tri.score_workspace_bytes(ctx, seqs) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tri.TriError) as e:
        tri.tri_score(ctx, seqs, scores, workspace=small)
    assert e.value.status == tri.TRI_E_INVAL


def test_gqa_deterministic_and_flat_and_nonfinite_rows(orc):
    """Two runs agree bit for bit; a head whose keys are all one row gets
    score 0 everywhere (every query head is flat); non-finite keys score NaN
    and drop out of the statistics of the others."""
    spec = synth.workload("gqa_toy").replace(lengths=(700,))
    cache = synth.make_cache(spec, "cuda", seed=5)
    k = cache.k[0]
    k[0, 0, :700] = k[0, 0, 3].clone()
    cache.pos[0][0, 0, :700] = 650          # same row and position: equal scores
    k[0, 1, 17, 5] = float("inf")
    k[0, 1, 301, 0] = float("nan")
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    a = torch.empty(2 * 700, device="cuda")
    b = torch.empty(2 * 700, device="cuda")
    tri.tri_score(ctx, seqs, a, workspace=ws)
    tri.tri_score(ctx, seqs, b, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
    sg = a.cpu().numpy().reshape(2, 700)
    assert np.all(sg[0] == 0.0)
    K, _, P = head_inputs(cache, 0, 0, 1)
    s_ref, tol = oracle_gqa(orc, cache, 0, 0, 1, K, P)
    assert np.isnan(sg[1, 17]) and np.isnan(sg[1, 301])
    check_agg(sg[1], s_ref, tol, "gqa non-finite keys")


@pytest.mark.parametrize("name,sample", [("gqa_small", None), ("qwen3_32k_gqa", [(0, 0), (35, 7)])])
def test_gqa_fused_pass(orc, name, sample):
    spec = synth.workload(name)
    B, W = spec.budget, spec.window
    say("gqa fused pass", name)
    cache = synth.make_cache(spec, "cuda", seed=6)
    n = cache.lens[0]
    pairs = sample or [(l, h) for l in range(spec.n_layers) for h in range(spec.n_kv_heads)]
    inputs = {(l, h): head_inputs(cache, 0, l, h) for l, h in pairs}
    k_in, v_in, p_in = cache.k[0].clone(), cache.v[0].clone(), cache.pos[0].clone()
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    scores = torch.empty(spec.heads * n, device="cuda")
    kept = torch.empty(spec.heads * B, dtype=torch.int32, device="cuda")
    tri.prune_step(ctx, seqs, B, W, scores, kept, workspace=ws)
    torch.cuda.synchronize()
    assert seqs[0].len == B
    check_topb_property(scores.view(spec.heads, n), kept.view(spec.heads, B), n)
    # compaction: rows r < B are the input rows at the GPU's kept list
    kl = kept.view(spec.n_layers, spec.n_kv_heads, B).long()
    for t_in, t_out in ((k_in, cache.k[0]), (v_in, cache.v[0])):
        g = torch.gather(t_in, 2, kl[..., None].expand(-1, -1, -1, spec.head_dim))
        assert torch.equal(bits(g), bits(t_out[:, :, :B]))
    assert torch.equal(torch.gather(p_in, 2, kl), cache.pos[0][:, :, :B])
    kg = kept.view(spec.n_layers, spec.n_kv_heads, B).cpu().numpy()
    for (l, h), (K, _, P) in inputs.items():
        s_ref, tol = oracle_gqa(orc, cache, 0, l, h, K, P)
        check_kept(orc, s_ref, tol, P, kg[l, h], B, W, "%s l%d h%d" % (name, l, h))


# ------------------------------------------- selection without the score array

@pytest.mark.parametrize("name,over", [
    ("gqa_toy", None), ("gqa_small", None), ("gqa_g7", None), ("gqa_g8_d64", None),
    ("gqa_small", {"dtype": "f32", "name": "gqa_small_f32"}),
    # two sequences of different lengths (the workspace sliced per sequence),
    # one that does not fire, and a length that ends inside a row group
    ("gqa_small", {"lengths": (4001, 300, 2600), "name": "gqa_small_three"}),
    # every register-resident length class (8, 16, 24 and 32 keys per thread)
    ("gqa_small", {"lengths": (20000, 9000, 30000, 5000), "name": "gqa_small_classes"}),
    # one past each class edge, and the largest head the register-resident path takes
    ("gqa_small", {"lengths": (8193, 16385, 24577, 32768, 24576), "name": "gqa_small_edges"}),
])
def test_gqa_select_from_the_workspace_equals_the_two_step_path(name, over):
    """tri_select_topb_ws (keys formed from the raw scores and statistics)
    keeps exactly the slots tri_select_topb keeps on the scores tri_score_ws
    writes: the same fp64 operations, rounded once."""
    spec = synth.workload(name)
    if over:
        spec = spec.replace(**over)
    B, W = min(spec.budget, 1000), 64
    say("gqa select from the workspace", spec.name, spec.lengths)
    cache = synth.make_cache(spec, "cuda", seed=21)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    total = sum(spec.heads * n for n in cache.lens)
    scores = torch.empty(total, device="cuda")
    kept_a = torch.full((spec.n_seq * spec.heads * B,), -5, dtype=torch.int32, device="cuda")
    kept_b = torch.full_like(kept_a, -5)
    tri.tri_score(ctx, seqs, scores, workspace=ws)
    tri.tri_select_topb(ctx, seqs, scores, B, W, kept_a)
    tri.tri_score(ctx, seqs, None, workspace=ws)
    tri.tri_select_topb_ws(ctx, seqs, ws, B, W, kept_b)
    torch.cuda.synchronize()
    assert torch.equal(kept_a, kept_b)
    fired = [tri.fires(q, B, W) for q in seqs]
    assert any(fired)
    say("  kept lists identical on %d sequences (%d fire)" % (len(seqs), sum(fired)))


def test_gqa_select_from_the_workspace_long_heads():
    """Heads longer than 32768 keys: the normalized scores go to the score
    array first (required then), and the kept lists still equal the two-step
    path's."""
    spec = synth.workload("gqa_toy").replace(name="gqa_long", lengths=(40000,))
    B, W = 3000, 128
    cache = synth.make_cache(spec, "cuda", seed=22)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    n = cache.lens[0]
    scores = torch.empty(spec.heads * n, device="cuda")
    scores_b = torch.empty_like(scores)
    kept_a = torch.empty(spec.heads * B, dtype=torch.int32, device="cuda")
    kept_b = torch.empty_like(kept_a)
    tri.tri_score(ctx, seqs, scores, workspace=ws)
    tri.tri_select_topb(ctx, seqs, scores, B, W, kept_a)
    tri.tri_score(ctx, seqs, None, workspace=ws)
    with pytest.raises(tri.TriError) as e:
        tri.tri_select_topb_ws(ctx, seqs, ws, B, W, kept_b)      # no score array
    assert e.value.status == tri.TRI_E_INVAL
    tri.tri_select_topb_ws(ctx, seqs, ws, B, W, kept_b, scores=scores_b)
    torch.cuda.synchronize()
    assert torch.equal(kept_a, kept_b)
    assert torch.equal(bits(scores), bits(scores_b))


def test_gqa_select_from_the_workspace_rejects_bad_arguments():
    spec = synth.workload("gqa_toy")
    cache = synth.make_cache(spec, "cuda", seed=23)
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    kept = torch.empty(spec.heads * 100, dtype=torch.int32, device="cuda")
    small = ws[:ws.numel() - 512]
    with pytest.raises(tri.TriError) as e:
        tri.tri_select_topb_ws(ctx, seqs, small, 100, 0, kept)
    assert e.value.status == tri.TRI_E_INVAL
    single = synth.workload("toy")
    c1 = synth.make_cache(single, "cuda", seed=24)
    ctx1 = tri.tri_calibrate_load(single.n_layers, single.n_kv_heads, single.head_dim, c1.calib.qc_re,
                                  c1.calib.qc_im, c1.calib.q_mean_norm, c1.calib.q_mrl, c1.calib.offsets,
                                  rope_theta=c1.calib.rope_theta, device=0)
    with pytest.raises(tri.TriError) as e:          # one query table per KV head: no GQA workspace
        tri.tri_select_topb_ws(ctx1, seqs_for(c1), ws, 100, 0, kept)
    assert e.value.status == tri.TRI_E_INVAL


@pytest.mark.parametrize("name,sample", [("gqa_small", None), ("qwen3_32k_gqa", [(0, 0), (17, 3), (35, 7)])])
def test_gqa_prune_step_without_scores(orc, name, sample):
    """The GQA prune step the benchmark times (score into the workspace,
    select from it, compact): kept sets against the oracle, the top-B of the
    GPU's own aggregated scores (taken by tri_score_ws on a copy), bit-exact
    compaction."""
    spec = synth.workload(name)
    B, W = spec.budget, spec.window
    say("gqa prune step without scores", name)
    cache = synth.make_cache(spec, "cuda", seed=6)
    n = cache.lens[0]
    pairs = sample or [(l, h) for l in range(spec.n_layers) for h in range(spec.n_kv_heads)]
    inputs = {(l, h): head_inputs(cache, 0, l, h) for l, h in pairs}
    k_in, v_in, p_in = cache.k[0].clone(), cache.v[0].clone(), cache.pos[0].clone()
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    scores = torch.empty(spec.heads * n, device="cuda")
    tri.tri_score(ctx, seqs, scores, workspace=ws)     # the GPU's own scores, for the property
    kept = torch.empty(spec.heads * B, dtype=torch.int32, device="cuda")
    tri.prune_step_gqa(ctx, seqs, B, W, kept, ws)
    torch.cuda.synchronize()
    assert seqs[0].len == B
    check_topb_property(scores.view(spec.heads, n), kept.view(spec.heads, B), n)
    kl = kept.view(spec.n_layers, spec.n_kv_heads, B).long()
    for t_in, t_out in ((k_in, cache.k[0]), (v_in, cache.v[0])):
        g = torch.gather(t_in, 2, kl[..., None].expand(-1, -1, -1, spec.head_dim))
        assert torch.equal(bits(g), bits(t_out[:, :, :B]))
    assert torch.equal(torch.gather(p_in, 2, kl), cache.pos[0][:, :, :B])
    kg = kept.view(spec.n_layers, spec.n_kv_heads, B).cpu().numpy()
    for (l, h), (K, _, P) in inputs.items():
        s_ref, tol = oracle_gqa(orc, cache, 0, l, h, K, P)
        check_kept(orc, s_ref, tol, P, kg[l, h], B, W, "%s l%d h%d" % (name, l, h))


def _random_gqa_spec(case):
    """A seeded small GQA configuration: G from 2 to 8 (every instantiated
    group size turns up), dtype, head_dim, layers, KV heads, one or two
    sequences, budget, window, RoPE base, offset set and key recipe."""
    rng = np.random.default_rng(2000 + case)
    recipe = ["toy", "concentrated", "phase"][int(rng.integers(3))]
    budget, window = int(rng.integers(1, 1200)), int(rng.integers(0, 200))
    lengths = tuple(int(x) for x in rng.integers(budget + window + 1, 5000, size=int(rng.integers(1, 3))))
    return synth.workload("gqa_small").replace(
        name="gqa_random%d" % case, group=2 + case % 7, n_layers=int(rng.integers(1, 3)),
        n_kv_heads=int(rng.integers(1, 3)), head_dim=[64, 128][int(rng.integers(2))],
        dtype=["bf16", "f32"][int(rng.integers(2))], rope_theta=float([1e4, 5e5, 1e6][int(rng.integers(3))]),
        lengths=lengths, budget=budget, window=window, recipe=recipe,
        offsets=synth.pow2_offsets(int(rng.integers(8, 17))),
        outlier_frac=0.05 if recipe == "concentrated" else 0.0)


@pytest.mark.parametrize("case", range(14))
def test_gqa_random_small_configs(orc, case):
    """Seeded random GQA configurations through the prune step the benchmark
    times (score into the workspace, select from it, compact): every head's
    kept set against the oracle, the top-B of the GPU's own aggregated scores,
    bit-exact compaction."""
    spec = _random_gqa_spec(case)
    B, W = spec.budget, spec.window
    say("gqa random config", case, "G =", spec.group, spec.dtype, spec.head_dim, spec.n_layers,
        spec.n_kv_heads, spec.lengths, B, W, spec.recipe)
    cache = synth.make_cache(spec, "cuda", seed=case)
    inputs = {(s, l, h): head_inputs(cache, s, l, h) for s in range(spec.n_seq)
              for l in range(spec.n_layers) for h in range(spec.n_kv_heads)}
    before = [(k.clone(), v.clone(), p.clone()) for k, v, p in zip(cache.k, cache.v, cache.pos)]
    ctx = ctx_gqa(cache)
    seqs = seqs_for(cache)
    ws = workspace_for(ctx, seqs)
    scores = torch.empty(tri.scores_count(ctx, seqs), device="cuda")
    tri.tri_score(ctx, seqs, scores, workspace=ws)     # the GPU's own scores, for the property
    kept = torch.empty(spec.n_seq * spec.heads * B, dtype=torch.int32, device="cuda")
    tri.prune_step_gqa(ctx, seqs, B, W, kept, ws)
    torch.cuda.synchronize()
    off = 0
    for s in range(spec.n_seq):
        n = cache.lens[s]
        assert seqs[s].len == B
        ks = kept[s * spec.heads * B:(s + 1) * spec.heads * B]
        check_topb_property(scores[off:off + spec.heads * n].view(spec.heads, n), ks.view(spec.heads, B), n)
        off += spec.heads * n
        kl = ks.view(spec.n_layers, spec.n_kv_heads, B).long()
        k_in, v_in, p_in = before[s]
        for t_in, t_out in ((k_in, cache.k[s]), (v_in, cache.v[s])):
            g = torch.gather(t_in, 2, kl[..., None].expand(-1, -1, -1, spec.head_dim))
            assert torch.equal(bits(g), bits(t_out[:, :, :B]))
        assert torch.equal(torch.gather(p_in, 2, kl), cache.pos[s][:, :, :B])
        kg = kl.cpu().numpy()
        for l in range(spec.n_layers):
            for h in range(spec.n_kv_heads):
                K, _, P = inputs[(s, l, h)]
                s_ref, tol = oracle_gqa(orc, cache, s, l, h, K, P)
                check_kept(orc, s_ref, tol, P, kg[l, h], B, W, "%s s%d l%d h%d" % (spec.name, s, l, h))
