"""GPU parity of head-specific budgets (the KV heads of a layer share
budget * n_kv_heads slots, every head keeping at least its `floor` best keys)
and of ragged caches (a length per head), through the C ABI, against the
fp64 oracle.

Bars:
  * shared select on synthetic fp32 scores: every kept list and count
    bit-exact with the oracle's, -1 counts for layers that do not fire.
  * compaction with per-head counts on oracle kept lists: K, V and positions
    bit-exact with the oracle's gather, head_len = count, heads with count -1
    untouched.
  * scores of a ragged cache: rows inside a head's length bit-identical to
    the scores of the same rows in a full cache, rows past it untouched; GQA
    scores of a ragged cache within the score bar of the oracle over the
    head's own rows.
  * fused prune step with shared budgets at the qwen3_32k shape: on every
    layer the GPU's kept sets satisfy the definition on the GPU's own scores
    (reserved keys kept, one layer threshold, ties to the lower head and
    slot, counts summing to the shared total), compacted rows are bit-exact
    copies of the input rows; on sampled layers the kept sets agree with the
    oracle's except for keys within 1e-4 * (M_i + M_t) of a threshold.
"""
import sys
import time

import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri

pytestmark = pytest.mark.gpu

TOL = 2e-3
TIGHT = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.load()


def dummy_ctx(L, H, d=64):
    z = np.zeros((L, H, d // 2))
    o = np.ones((L, H, d // 2))
    return tri.tri_calibrate_load(L, H, d, z, z, o, o, [1], device=0)


def run_shared(ctx, L, H, n, sc, hl, budget, floor, window):
    """GPU shared select on host fp32 scores [L][H][n] and head lengths."""
    total = budget * H
    k = torch.zeros((L, H, n, 64), dtype=torch.float32, device="cuda")
    head_len = torch.from_numpy(hl).cuda() if hl is not None else None
    seq = tri.Seq(k, None, None, n, n - 1, head_len)
    kept = torch.full((L * H * total,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((L * H,), -9, dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, 1), dtype=torch.uint8, device="cuda")
    tri.tri_select_shared(ctx, [seq], torch.from_numpy(sc.reshape(-1)).cuda(), budget, floor,
                          window, kept, counts, ws)
    torch.cuda.synchronize()
    return kept.cpu().numpy().reshape(L, H, total), counts.cpu().numpy().reshape(L, H)


def check_layer_vs_oracle(orc, sc_l, lens, kept_l, counts_l, total, floor, window, what):
    H, n = sc_l.shape
    pos = np.broadcast_to(np.arange(n), (H, n))
    ref = orc.select_shared(sc_l.astype(np.float64), pos, lens, total, floor, window)
    if ref is None:
        assert np.all(counts_l == -1), what + ": a layer that does not fire got counts"
        assert np.all(kept_l == -7) or floor > 0, what
        return False
    for h in range(H):
        c = int(counts_l[h])
        assert c == len(ref[h]), "%s head %d: count %d, oracle %d" % (what, h, c, len(ref[h]))
        np.testing.assert_array_equal(kept_l[h, :c], ref[h], err_msg="%s head %d" % (what, h))
    assert int(counts_l.sum()) == total
    return True


SHARED_CASES = [
    # kind, L, H, n, budget, floor, window, lengths
    ("normal", 2, 8, 5000, 512, 64, 0, "full"),
    ("ties", 2, 8, 3000, 256, 32, 0, "ragged"),
    ("allequal", 1, 4, 2000, 300, 100, 0, "full"),
    ("special", 2, 8, 4096, 512, 128, 16, "ragged"),
    ("dups", 1, 8, 9000, 1024, 0, 0, "full"),
    ("straddle", 2, 8, 32768, 4096, 256, 128, "full"),
    ("narrow", 1, 8, 7000, 800, 800, 0, "ragged"),
    ("ulp", 2, 3, 40000, 2000, 100, 0, "ragged"),
    ("outlier", 1, 8, 1000, 100, 20, 0, "full"),
    ("normal", 3, 8, 1000, 100, 40, 0, "extreme"),
    ("ties", 3, 8, 600, 64, 64, 0, "extreme"),
    ("normal", 1, 1, 3000, 700, 10, 0, "full"),
    ("normal", 2, 5, 129, 1, 1, 0, "ragged"),
    ("normal", 2, 128, 300, 20, 5, 0, "ragged"),
    ("wide", 2, 8, 20000, 2048, 256, 0, "ragged"),
]


@pytest.mark.parametrize("kind,L,H,n,budget,floor,window,lengths", SHARED_CASES)
def test_shared_select_bit_exact_on_synthetic_scores(orc, kind, L, H, n, budget, floor, window,
                                                     lengths):
    say("shared select", kind, L, H, n, budget, floor, window, lengths)
    sc = synth.make_scores(kind, L * H, n, seed=n + H).reshape(L, H, n)
    hl = synth.head_lengths(lengths, L, H, n, seed=L * 7 + H)
    ctx = dummy_ctx(L, H)
    kept, counts = run_shared(ctx, L, H, n, sc, hl, budget, floor, window)
    fired = 0
    for l in range(L):
        fired += check_layer_vs_oracle(orc, sc[l], hl[l], kept[l], counts[l], budget * H, floor,
                                       window, "layer %d" % l)
    say("  layers fired: %d of %d" % (fired, L))


def _random_shared_case(case):
    """A seeded draw of score kind, layers, KV heads, keys per head, budget,
    floor, window and head lengths for the shared selection."""
    rng = np.random.default_rng(3000 + case)
    kinds = ["normal", "ties", "allequal", "special", "dups", "straddle", "narrow", "ulp",
             "outlier", "wide"]
    L, H = int(rng.integers(1, 4)), int(rng.integers(1, 17))
    n = int(rng.integers(50, 20000))
    budget = int(rng.integers(1, max(2, n // 2)))
    floor = int(rng.integers(0, budget + 1))
    window = int(rng.integers(0, 100))
    lengths = ["full", "ragged", "extreme"][int(rng.integers(3))]
    return kinds[int(rng.integers(len(kinds)))], L, H, n, budget, floor, window, lengths


@pytest.mark.parametrize("case", range(20))
def test_shared_select_random_synthetic_scores(orc, case):
    """Seeded random shared selections on synthetic scores, bit-exact with the
    oracle's shared selection on every layer."""
    kind, L, H, n, budget, floor, window, lengths = _random_shared_case(case)
    test_shared_select_bit_exact_on_synthetic_scores(orc, kind, L, H, n, budget, floor, window,
                                                     lengths)


def test_shared_select_without_head_lengths(orc):
    """head_len NULL: every head holds len rows."""
    L, H, n, B, F = 2, 8, 4000, 300, 30
    sc = synth.make_scores("dups", L * H, n, seed=5).reshape(L, H, n)
    ctx = dummy_ctx(L, H)
    kept, counts = run_shared(ctx, L, H, n, sc, None, B, F, 0)
    for l in range(L):
        assert check_layer_vs_oracle(orc, sc[l], np.full(H, n), kept[l], counts[l], B * H, F, 0,
                                     "layer %d" % l)


def test_shared_select_firing_rule(orc):
    """A layer fires iff the sum of its heads' lengths exceeds total + H * window."""
    L, H, n, B, W = 3, 4, 500, 100, 20
    hl = np.array([[120, 120, 120, 120],      # 480 = 400 + 80: does not fire
                   [121, 120, 120, 120],      # 481: fires
                   [500, 0, 0, 0]], dtype=np.int32)
    sc = synth.make_scores("normal", L * H, n, seed=3).reshape(L, H, n)
    ctx = dummy_ctx(L, H)
    kept, counts = run_shared(ctx, L, H, n, sc, hl, B, 10, W)
    assert np.all(counts[0] == -1)
    for l in (1, 2):
        assert check_layer_vs_oracle(orc, sc[l], hl[l], kept[l], counts[l], B * H, 10, W,
                                     "layer %d" % l)


def test_shared_floor_equal_to_budget_is_the_uniform_select(orc):
    """floor = budget: every head keeps exactly its own top-budget keys."""
    L, H, n, B = 2, 8, 6000, 700
    sc = synth.make_scores("ties", L * H, n, seed=8).reshape(L, H, n)
    ctx = dummy_ctx(L, H)
    kept, counts = run_shared(ctx, L, H, n, sc, None, B, B, 0)
    assert np.all(counts == B)
    for l in range(L):
        for h in range(H):
            np.testing.assert_array_equal(kept[l, h, :B], orc.select_head(
                sc[l, h].astype(np.float64), np.arange(n), B, 0))


def test_uniform_calls_reject_ragged_caches():
    ctx = dummy_ctx(1, 2)
    k = torch.zeros((1, 2, 100, 64), device="cuda")
    v = torch.zeros_like(k)
    p = torch.zeros((1, 2, 100), dtype=torch.int32, device="cuda")
    hl = torch.full((1, 2), 100, dtype=torch.int32, device="cuda")
    seq = tri.Seq(k, v, p, 100, 99, hl)
    sc = torch.zeros(200, device="cuda")
    kept = torch.zeros(200, dtype=torch.int32, device="cuda")
    with pytest.raises(tri.TriError):
        tri.tri_select_topb(ctx, [seq], sc, 10, 0, kept)
    with pytest.raises(tri.TriError):
        tri.tri_compact_kv(ctx, [seq], kept, 10, 0)
    seq.head_len = None
    with pytest.raises(tri.TriError):     # the counted compaction needs head lengths
        tri.tri_compact_kv_counts(ctx, [seq], kept, 10, kept[:2], kept)


# ------------------------------------------------------------ compaction

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_compact_counts_bit_exact(orc, dtype, d):
    L, H, n, B, F = 3, 8, 5000, 400, 50
    total = B * H
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + d)
    K = torch.randn((L, H, n + 5, d), generator=g, device="cuda").to(tdt)
    V = torch.randn((L, H, n + 5, d), generator=g, device="cuda").to(tdt)
    P = (torch.arange(n + 5, dtype=torch.int32, device="cuda") * 3 + 7).repeat(L, H, 1)
    K0, V0, P0 = K.cpu(), V.cpu(), P.cpu()
    hl = synth.head_lengths("ragged", L, H, n, seed=d)
    hl[2] = 100                                 # layer 2 does not fire
    sc = synth.make_scores("dups", L * H, n, seed=d).reshape(L, H, n)
    kept = np.full((L, H, total), -1, dtype=np.int32)
    counts = np.full((L, H), -1, dtype=np.int32)
    refs = []
    for l in range(L):
        r = orc.select_shared(sc[l].astype(np.float64), P0[l].numpy()[:, :n].astype(np.int64),
                              hl[l], total, F, 0)
        refs.append(r)
        if r is not None:
            for h in range(H):
                counts[l, h] = len(r[h])
                kept[l, h, :len(r[h])] = r[h]
    assert refs[2] is None and refs[0] is not None
    ctx = tri.tri_calibrate_load(L, H, d, np.zeros((L, H, d // 2)), np.zeros((L, H, d // 2)),
                                 np.ones((L, H, d // 2)), np.ones((L, H, d // 2)), [1], device=0)
    head_len = torch.from_numpy(hl).cuda()
    seq = tri.Seq(K, V, P, n, n - 1, head_len)
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")
    tri.tri_compact_kv_counts(ctx, [seq], torch.from_numpy(kept).cuda().reshape(-1), total,
                              torch.from_numpy(counts).cuda().reshape(-1), cws)
    torch.cuda.synchronize()
    assert seq.len == n
    hl_after = head_len.cpu().numpy()
    Kc, Vc, Pc = K.cpu(), V.cpu(), P.cpu()
    raw = lambda t: t.contiguous().view(torch.uint8).numpy()
    for l in range(L):
        for h in range(H):
            if refs[l] is None:
                assert hl_after[l, h] == hl[l, h]
                assert torch.equal(Kc[l, h].view(torch.uint8), K0[l, h].view(torch.uint8))
                assert torch.equal(Vc[l, h].view(torch.uint8), V0[l, h].view(torch.uint8))
                assert torch.equal(Pc[l, h], P0[l, h])
                continue
            kk = refs[l][h]
            c = len(kk)
            assert hl_after[l, h] == c
            np.testing.assert_array_equal(raw(Kc[l, h, :c]), orc.gather_rows(kk, raw(K0[l, h, :n])))
            np.testing.assert_array_equal(raw(Vc[l, h, :c]), orc.gather_rows(kk, raw(V0[l, h, :n])))
            np.testing.assert_array_equal(Pc[l, h, :c].numpy(), orc.gather_rows(kk, P0[l, h, :n].numpy()))


# ------------------------------------------------------- ragged scoring

def ctx_for(cache):
    sp, cal = cache.spec, cache.calib
    return tri.tri_calibrate_load(sp.n_layers, sp.n_kv_heads, sp.head_dim, cal.qc_re, cal.qc_im,
                                  cal.q_mean_norm, cal.q_mrl, cal.offsets,
                                  rope_theta=cal.rope_theta, device=0,
                                  n_q_heads=sp.n_q_heads)


def test_ragged_scores_equal_full_scores_inside_each_head():
    spec = synth.workload("llama8b").replace(name="ragged", n_layers=3, lengths=(5000,))
    cache = synth.make_cache(spec, "cuda", seed=21)
    H, n = spec.heads, 5000
    ctx = ctx_for(cache)
    full = torch.empty(H * n, device="cuda")
    tri.tri_score(ctx, [tri.Seq(cache.k[0], None, None, n, cache.p_now[0])], full)
    hl = synth.head_lengths("extreme", spec.n_layers, spec.n_kv_heads, n, seed=2)
    rag = torch.full((H * n,), 12345.0, device="cuda")
    tri.tri_score(ctx, [tri.Seq(cache.k[0], None, None, n, cache.p_now[0],
                                torch.from_numpy(hl).cuda())], rag)
    torch.cuda.synchronize()
    f = full.view(H, n).cpu().numpy()
    r = rag.view(H, n).cpu().numpy()
    for i, m in enumerate(hl.reshape(-1)):
        np.testing.assert_array_equal(r[i, :m].view(np.int32), f[i, :m].view(np.int32))
        assert np.all(r[i, m:] == 12345.0)


@pytest.mark.parametrize("name", ["gqa_small", "gqa_g8_d64"])
def test_ragged_gqa_scores_against_the_oracle(orc, name):
    """Per-query-head statistics over each head's own rows only (the bar of
    the full-cache GQA parity test, derived there)."""
    from test_gpu_gqa import check_agg, oracle_gqa
    spec = synth.workload(name)
    cache = synth.make_cache(spec, "cuda", seed=5)
    H, n = spec.heads, cache.lens[0]
    hl = synth.head_lengths("extreme", spec.n_layers, spec.n_kv_heads, n, seed=9)
    hl.reshape(-1)[0] = n
    ctx = ctx_for(cache)
    seq = tri.Seq(cache.k[0], None, None, n, cache.p_now[0], torch.from_numpy(hl).cuda())
    scores = torch.full((H * n,), 777.0, device="cuda")
    ws = torch.empty(tri.score_workspace_bytes(ctx, [seq]), dtype=torch.uint8, device="cuda")
    tri.tri_score(ctx, [seq], scores, workspace=ws)
    torch.cuda.synchronize()
    sg = scores.view(H, n).cpu().numpy()
    for l in range(spec.n_layers):
        for h in range(spec.n_kv_heads):
            m = int(hl[l, h])
            hi = l * spec.n_kv_heads + h
            assert np.all(sg[hi, m:] == 777.0)
            if m == 0:
                continue
            K = cache.k[0][l, h, :m].float().cpu().numpy()
            P = cache.pos[0][l, h, :m].cpu().numpy()
            s_ref, tol = oracle_gqa(orc, cache, 0, l, h, K, P)
            check_agg(sg[hi, :m], s_ref, tol, "l%d h%d (%d rows)" % (l, h, m))


# ------------------------------------------------------------ fused pass

def check_shared_property(sc, kept, counts, lens, total, floor):
    """GPU-internal: on one layer the kept sets are the shared-budget choice
    for the GPU's own scores (finite scores)."""
    H, n = sc.shape
    assert int(counts.sum()) == total
    in_layer = []
    for h in range(H):
        c, m = int(counts[h]), int(lens[h])
        kk = kept[h, :c].astype(np.int64)
        assert c >= min(m, floor)
        assert np.all(np.diff(kk) > 0) and (c == 0 or (kk[0] >= 0 and kk[-1] < m))
        s = sc[h, :m].astype(np.float64)
        assert np.all(np.isfinite(s))
        order = np.lexsort((np.arange(m), -s))
        res = np.zeros(m, bool)
        res[order[:min(m, floor)]] = True
        sel = np.zeros(m, bool)
        sel[kk] = True
        assert sel[res].all(), "head %d: a reserved key was evicted" % h
        in_layer.append((s, res, sel))
    kept_min, ev_max = np.inf, -np.inf
    for s, res, sel in in_layer:
        if (sel & ~res).any():
            kept_min = min(kept_min, s[sel & ~res].min())
        if (~sel).any():
            ev_max = max(ev_max, s[~sel].max())
    assert kept_min >= ev_max, "an evicted key outscores a kept unreserved key"
    if kept_min == ev_max:
        # equal keys straddle: every kept one precedes every evicted one in
        # (head, slot) order
        last_kept, first_ev = (-1, -1), (H, 0)
        for h, (s, res, sel) in enumerate(in_layer):
            at = s == kept_min
            ks = np.nonzero(at & sel & ~res)[0]
            es = np.nonzero(at & ~sel)[0]
            if len(ks):
                last_kept = max(last_kept, (h, int(ks[-1])))
            if len(es):
                first_ev = min(first_ev, (h, int(es[0])))
        assert last_kept < first_ev


def oracle_layer(orc, cache, l, K, P, lens):
    """Oracle scores of one layer's heads over their own rows, with the
    per-key score tolerance (TOL * M for one query table per head, the
    derived GQA bar otherwise)."""
    sp, cal = cache.spec, cache.calib
    H1, n = K.shape[0], K.shape[1]
    s_ref = np.full((H1, n), -np.inf)
    tol = np.zeros((H1, n))
    om = orc.omega(sp.head_dim, sp.rope_theta)
    for h in range(H1):
        m = int(lens[h])
        if m == 0:
            continue
        if sp.group > 1:
            from test_gpu_gqa import oracle_gqa
            s_ref[h, :m], tol[h, :m] = oracle_gqa(orc, cache, 0, l, h, K[h, :m], P[h, :m])
        else:
            args = (cal.qc_re[l, h], cal.qc_im[l, h], cal.q_mean_norm[l, h], cal.q_mrl[l, h])
            _, _, s_ref[h, :m] = orc.score_head(K[h, :m], P[h, :m], cache.p_now[0], om,
                                                cal.offsets, *args)
            tol[h, :m] = TOL * orc.bound_head(K[h, :m], om, cal.offsets, *args)
    return s_ref, tol


def fused_shared(orc, spec, seed, lengths, floor, sample):
    """One shared-budget prune step (score, shared select, counted compaction)
    in the benchmark's launch configuration, checked on every layer against
    the definition on the GPU's own scores and on sampled layers against the
    oracle."""
    L, H1, n, B, W = spec.n_layers, spec.n_kv_heads, spec.lengths[0], spec.budget, spec.window
    total = B * H1
    t0 = time.time()
    say("fused shared %s: lengths %s, floor %d" % (spec.name, lengths, floor))
    cache = synth.make_cache(spec, "cuda", seed=seed)
    hl = synth.head_lengths(lengths, L, H1, n, seed=seed)
    ins = {l: (cache.k[0][l].float().cpu().numpy(), cache.pos[0][l].cpu().numpy()) for l in sample}
    K0, V0, P0 = cache.k[0].clone(), cache.v[0].clone(), cache.pos[0].clone()
    ctx = ctx_for(cache)
    head_len = torch.from_numpy(hl).cuda()
    seq = tri.Seq(cache.k[0], cache.v[0], cache.pos[0], n, cache.p_now[0], head_len)
    scores = torch.empty(L * H1 * n, device="cuda")
    kept = torch.full((L * H1 * total,), -1, dtype=torch.int32, device="cuda")
    counts = torch.empty((L * H1,), dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, 1), dtype=torch.uint8, device="cuda")
    sws = None
    if spec.group > 1:
        sws = torch.empty(tri.score_workspace_bytes(ctx, [seq]), dtype=torch.uint8, device="cuda")
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")
    tri.prune_step_shared(ctx, [seq], B, floor, W, scores, kept, counts, ws, cws, workspace=sws)
    torch.cuda.synchronize()
    say("  shared prune step done, %.1fs" % (time.time() - t0))
    sc = scores.view(L, H1, n).cpu().numpy()
    kp = kept.view(L, H1, total).cpu().numpy()
    ct = counts.view(L, H1).cpu().numpy()
    hl_after = head_len.cpu().numpy()
    spread, fired = [], []
    for l in range(L):
        if hl[l].sum() <= total + H1 * W:
            assert np.all(ct[l] == -1) and np.array_equal(hl_after[l], hl[l])
            fired.append(False)
            continue
        fired.append(True)
        assert np.array_equal(hl_after[l], ct[l])
        check_shared_property(sc[l], kp[l], ct[l], hl[l], total, floor)
        spread.append(ct[l].max() - ct[l].min())
        idx = torch.from_numpy(kp[l]).cuda().long()
        for h in range(H1):
            c = int(ct[l, h])
            ii = idx[h, :c]
            assert torch.equal(bits(cache.k[0][l, h, :c]), bits(K0[l, h, ii]))
            assert torch.equal(bits(cache.v[0][l, h, :c]), bits(V0[l, h, ii]))
            assert torch.equal(cache.pos[0][l, h, :c], P0[l, h, ii])
    say("  layers fired %d of %d; counts spread within a layer: max %d, mean %.1f"
        % (sum(fired), L, max(spread), float(np.mean(spread))))
    for l in sample:
        K, P = ins[l]
        s_ref, tol = oracle_layer(orc, cache, l, K, P, hl[l])
        for h in range(H1):
            m = int(hl[l, h])
            err = np.abs(sc[l, h, :m].astype(np.float64) - s_ref[h, :m])
            assert np.all(err <= tol[h, :m]), "layer %d head %d: score bar" % (l, h)
        if not fired[l]:
            continue
        ref = orc.select_shared(s_ref, P.astype(np.int64), hl[l], total, floor, W)
        assert ref is not None
        # thresholds of the oracle's choice: each head's floor-th score and the
        # layer's last admitted unreserved score
        t_h = np.full(H1, np.nan)
        res = np.zeros((H1, n), bool)
        sel_ref = np.zeros((H1, n), bool)
        for h in range(H1):
            m = int(hl[l, h])
            order = np.lexsort((P[h, :m], -s_ref[h, :m]))
            if m > floor and floor > 0:
                t_h[h] = s_ref[h, order[floor - 1]]
            res[h, order[:min(m, floor)]] = True
            sel_ref[h, ref[h]] = True
        free = sel_ref & ~res
        t = s_ref[free].min() if free.any() else np.nan
        tol_max = tol.max()
        ndis = 0
        for h in range(H1):
            sel = np.zeros(n, bool)
            sel[kp[l, h, :int(ct[l, h])]] = True
            dis = np.nonzero(sel != sel_ref[h])[0]
            ndis += len(dis)
            if len(dis):
                band = (TIGHT / TOL) * (tol[h, dis] + tol_max)
                near = (np.abs(s_ref[h, dis] - t) <= band) | (np.abs(s_ref[h, dis] - t_h[h]) <= band)
                assert near.all(), "layer %d head %d: a clear disagreement" % (l, h)
        say("  layer %d: kept-set disagreements with the oracle: %d of %d" % (l, ndis, total))
    del cache, K0, V0, P0, scores, kept
    torch.cuda.empty_cache()


def bits(t):
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])


def test_fused_shared_qwen3_32k_full(orc):
    """The benchmark's shared-budget configuration: qwen3_32k, floor = budget / 4."""
    spec = synth.workload("qwen3_32k")
    fused_shared(orc, spec, 0, "full", spec.budget // 4, (0, 35))


def test_fused_shared_ragged_llama8b(orc):
    """A ragged cache (as an earlier shared prune leaves it), every layer checked
    against the oracle."""
    spec = synth.workload("llama8b").replace(name="ragged8b", n_layers=4, lengths=(8192,))
    fused_shared(orc, spec, 3, "ragged", 256, (0, 1, 2, 3))


def test_fused_shared_extreme_lengths(orc):
    spec = synth.workload("llama8b").replace(name="extreme8b", n_layers=4, lengths=(6000,),
                                             budget=700)
    fused_shared(orc, spec, 4, "extreme", 100, (0, 1, 2, 3))


def test_fused_shared_gqa(orc):
    spec = synth.workload("gqa_small")
    fused_shared(orc, spec, 2, "ragged", spec.budget // 8, tuple(range(spec.n_layers)))


@pytest.mark.parametrize("case", range(10))
def test_fused_shared_random_small_configs(orc, case):
    """Seeded random small caches through the shared-budget prune step (single
    table or GQA), every layer against the oracle and every compacted row bit
    for bit."""
    rng = np.random.default_rng(4000 + case)
    recipe = ["toy", "concentrated", "phase", "neartie"][int(rng.integers(4))]
    group = int(rng.choice([1, 1, 2, 4]))
    dtype = "bf16" if recipe == "neartie" or group > 1 else ["bf16", "f32"][int(rng.integers(2))]
    n = int(rng.integers(300, 6000))
    budget = int(rng.integers(16, max(17, n // 3)))
    spec = synth.workload("llama8b").replace(
        name="shared_random%d" % case, n_layers=int(rng.integers(1, 4)),
        n_kv_heads=int(rng.integers(1, 9)), head_dim=[64, 128][int(rng.integers(2))], dtype=dtype,
        rope_theta=float([1e4, 5e5, 1e6][int(rng.integers(3))]), lengths=(n,), budget=budget,
        window=int(rng.integers(0, 150)), recipe=recipe, group=group,
        offsets=synth.pow2_offsets(int(rng.integers(8, 17))),
        dup_frac=0.1 if recipe == "neartie" else 0.0,
        outlier_frac=0.05 if recipe == "concentrated" else 0.0)
    floor = int(rng.integers(0, budget + 1))
    lengths = ["full", "ragged", "extreme"][int(rng.integers(3))]
    fused_shared(orc, spec, case, lengths, floor, tuple(range(spec.n_layers)))


def test_shared_select_and_compaction_over_several_sequences(orc):
    """Three sequences of different lengths (one that fires nowhere) in one
    call: the workspace slices per sequence, the kept and count layouts, and
    the counted compaction's reused queue."""
    L, H, B, F, W = 2, 8, 300, 40, 16
    lens = [3000, 2500, 200]
    total = B * H
    ctx = dummy_ctx(L, H, d=64)
    seqs, hls, scs, pristine = [], [], [], []
    for s, n in enumerate(lens):
        g = torch.Generator(device="cuda")
        g.manual_seed(77 + s)
        K = torch.randn((L, H, n, 64), generator=g, device="cuda")
        V = torch.randn((L, H, n, 64), generator=g, device="cuda")
        P = torch.arange(n, dtype=torch.int32, device="cuda").repeat(L, H, 1)
        hl = synth.head_lengths("ragged", L, H, n, seed=s)
        hls.append(hl)
        scs.append(synth.make_scores("dups", L * H, n, seed=s).reshape(L, H, n))
        pristine.append((K.cpu(), V.cpu(), P.cpu()))
        seqs.append(tri.Seq(K, V, P, n, n - 1, torch.from_numpy(hl).cuda()))
    scores = torch.from_numpy(np.concatenate([x.reshape(-1) for x in scs])).cuda()
    kept = torch.full((len(lens) * L * H * total,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((len(lens) * L * H,), -9, dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, len(lens)), dtype=torch.uint8,
                     device="cuda")
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")
    tri.tri_select_shared(ctx, seqs, scores, B, F, W, kept, counts, ws)
    kept_h = kept.cpu().numpy().reshape(len(lens), L, H, total)
    cnt_h = counts.cpu().numpy().reshape(len(lens), L, H)
    tri.tri_compact_kv_counts(ctx, seqs, kept, total, counts, cws)
    torch.cuda.synchronize()
    for s, n in enumerate(lens):
        K0, V0, P0 = pristine[s]
        hl_after = seqs[s].head_len.cpu().numpy()
        for l in range(L):
            pos = np.broadcast_to(np.arange(n), (H, n))
            ref = orc.select_shared(scs[s][l].astype(np.float64), pos, hls[s][l], total, F, W)
            if ref is None:
                assert np.all(cnt_h[s, l] == -1)
                assert np.array_equal(hl_after[l], hls[s][l])
                continue
            for h in range(H):
                c = len(ref[h])
                assert cnt_h[s, l, h] == c and hl_after[l, h] == c
                np.testing.assert_array_equal(kept_h[s, l, h, :c], ref[h])
                kk = torch.from_numpy(ref[h]).long()
                assert torch.equal(seqs[s].k[l, h, :c].cpu(), K0[l, h, kk])
                assert torch.equal(seqs[s].v[l, h, :c].cpu(), V0[l, h, kk])
                assert torch.equal(seqs[s].pos[l, h, :c].cpu(), P0[l, h, kk])
    assert cnt_h[2].max() == -1        # 8 heads of <= 200 keys never exceed 8 x 300 + 8 x 16


def test_shared_calls_reject_bad_arguments():
    L, H, n = 1, 4, 500
    ctx = dummy_ctx(L, H)
    k = torch.zeros((L, H, n, 64), device="cuda")
    hl = torch.full((L, H), n, dtype=torch.int32, device="cuda")
    seq = tri.Seq(k, torch.zeros_like(k), torch.zeros((L, H, n), dtype=torch.int32, device="cuda"),
                  n, n - 1, hl)
    sc = torch.zeros(L * H * n, device="cuda")
    kept = torch.zeros(L * H * 100 * H, dtype=torch.int32, device="cuda")
    counts = torch.zeros(L * H, dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, 1), dtype=torch.uint8, device="cuda")
    lib = tri.library()
    arr = (tri._Seq * 1)(tri._Seq(k.data_ptr(), seq.v.data_ptr(), seq.pos.data_ptr(), n, n, n - 1,
                                  hl.data_ptr()))
    call = lambda budget, floor, window, wsb, kc=counts.data_ptr(): lib.tri_select_shared(
        ctx.handle, arr, 1, sc.data_ptr(), budget, floor, window, kept.data_ptr(), kc,
        ws.data_ptr(), wsb, None)
    nb = ws.numel()
    assert call(100, 101, 0, nb) == tri.TRI_E_INVAL          # floor above the budget
    assert call(100, -1, 0, nb) == tri.TRI_E_INVAL           # negative floor
    assert call(0, 0, 0, nb) == tri.TRI_E_INVAL              # no budget
    assert call(100, 10, -1, nb) == tri.TRI_E_INVAL          # negative window
    assert call(100, 10, 0, nb - 1) == tri.TRI_E_INVAL       # short workspace
    assert call(100, 10, 0, nb, kc=None) == tri.TRI_E_INVAL  # no counts
    assert call(100, 10, 0, nb) == tri.TRI_OK
    big = dummy_ctx(1, 129)
    assert lib.tri_select_shared(big.handle, arr, 0, None, 1, 0, 0, None, None, None, 0,
                                 None) == tri.TRI_E_UNSUPPORTED
    torch.cuda.synchronize()


def test_shared_prune_then_append_then_prune(orc):
    """Two prune cycles with head-specific budgets and a decode window between
    them: after the first prune the heads hold different lengths; 128 new
    keys are appended to every head at its own length; the second prune runs
    on that ragged cache.  Every step is replayed by the oracle from the same
    inputs (its own scores, selection and gather), and the final K, V,
    positions and lengths are compared bit for bit."""
    L, H1, n, W, B, F = 2, 8, 3000, 128, 256, 32
    total = B * H1
    spec = synth.workload("llama8b").replace(name="append", n_layers=L, lengths=(n, W))
    pos_new = np.arange(n, n + W)
    cache = synth.make_cache(spec, "cuda", seed=8, positions=[np.arange(n), pos_new],
                             p_now=[n - 1, n + W - 1], caps=[n + W, W])
    cal = cache.calib
    om = orc.omega(spec.head_dim, spec.rope_theta)
    K, V, P = cache.k[0], cache.v[0], cache.pos[0]
    Kn, Vn = cache.k[1][:, :, :W].clone(), cache.v[1][:, :, :W].clone()
    host = {"K": K[:, :, :n].float().cpu().numpy(), "Kb": K[:, :, :n].cpu(),
            "V": V[:, :, :n].cpu(), "P": P[:, :, :n].cpu().numpy()}
    Kn_f, Kn_b, Vn_h = Kn.float().cpu().numpy(), Kn.cpu(), Vn.cpu()
    ctx = ctx_for(cache)
    head_len = torch.full((L, H1), n, dtype=torch.int32, device="cuda")
    kept = torch.empty(L * H1 * total, dtype=torch.int32, device="cuda")
    counts = torch.empty(L * H1, dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, 1), dtype=torch.uint8, device="cuda")
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")

    def gpu_prune(length, p_now):
        seq = tri.Seq(K, V, P, length, p_now, head_len)
        scores = torch.empty(L * H1 * length, device="cuda")
        tri.prune_step_shared(ctx, [seq], B, F, 0, scores, kept, counts, ws, cws)
        torch.cuda.synchronize()

    def oracle_prune(rows_f, rows_k, rows_v, rows_p, p_now, l):
        """rows_*[h]: the head's rows (fp32 view, stored dtype, V, positions)."""
        lens = [len(r) for r in rows_p]
        stride = max(lens)
        S = np.full((H1, stride), -np.inf)
        Pm = np.zeros((H1, stride), dtype=np.int64)
        for h in range(H1):
            args = (cal.qc_re[l, h], cal.qc_im[l, h], cal.q_mean_norm[l, h], cal.q_mrl[l, h])
            _, _, S[h, :lens[h]] = orc.score_head(rows_f[h], rows_p[h], p_now, om, cal.offsets, *args)
            Pm[h, :lens[h]] = rows_p[h]
        sel = orc.select_shared(S, Pm, lens, total, F, 0)
        assert sel is not None
        take = lambda x, k: x[torch.from_numpy(k).long()] if torch.is_tensor(x) else x[k]
        return ([take(rows_f[h], sel[h]) for h in range(H1)], [take(rows_k[h], sel[h]) for h in range(H1)],
                [take(rows_v[h], sel[h]) for h in range(H1)], [take(rows_p[h], sel[h]) for h in range(H1)])

    # first prune
    gpu_prune(n, n - 1)
    hl1 = head_len.cpu().numpy().copy()
    # decode window: 128 new keys per head at the head's own length
    for l in range(L):
        for h in range(H1):
            c = int(hl1[l, h])
            K[l, h, c:c + W] = Kn[l, h]
            V[l, h, c:c + W] = Vn[l, h]
            P[l, h, c:c + W] = torch.from_numpy(pos_new).to(torch.int32).cuda()
    head_len += W
    assert int(head_len.max()) <= n + W
    # second prune on the ragged cache
    gpu_prune(n + W, n + W - 1)
    hl2 = head_len.cpu().numpy()

    for l in range(L):
        f1, k1, v1, p1 = oracle_prune([host["K"][l, h] for h in range(H1)],
                                      [host["Kb"][l, h] for h in range(H1)],
                                      [host["V"][l, h] for h in range(H1)],
                                      [host["P"][l, h] for h in range(H1)], n - 1, l)
        assert [len(x) for x in p1] == list(hl1[l]), "layer %d: first-prune counts" % l
        f2in = [np.concatenate([f1[h], Kn_f[l, h]]) for h in range(H1)]
        k2in = [torch.cat([k1[h], Kn_b[l, h]]) for h in range(H1)]
        v2in = [torch.cat([v1[h], Vn_h[l, h]]) for h in range(H1)]
        p2in = [np.concatenate([p1[h], pos_new]) for h in range(H1)]
        _, k2, v2, p2 = oracle_prune(f2in, k2in, v2in, p2in, n + W - 1, l)
        for h in range(H1):
            c = len(p2[h])
            assert hl2[l, h] == c, "layer %d head %d: final count" % (l, h)
            np.testing.assert_array_equal(P[l, h, :c].cpu().numpy(), p2[h])
            assert torch.equal(K[l, h, :c].cpu().view(torch.int16), k2[h].view(torch.int16))
            assert torch.equal(V[l, h, :c].cpu().view(torch.int16), v2[h].view(torch.int16))
    say("  two prune cycles agree with the oracle on every head; lengths after the first prune %s"
        % sorted(set(hl1.reshape(-1).tolist()))[:6])
