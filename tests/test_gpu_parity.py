"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle.

Bars:
  * scores: |s_gpu - s_ref| <= 2e-3 * M_i for every compared key, with M_i
    the oracle's per-key magnitude bound (the scale of any evaluation's
    rounding error); the observed maximum is printed and is ~1e-6.
  * select on synthetic fp32 scores: kept lists bit-exact with the oracle.
  * compact on synthetic kept lists: K, V and positions bit-exact with the
    oracle's gather.
  * fused pass: every key the oracle ranks above its B-th score t by more than
    tau_i = 2e-3 * (M_i + M_t) is kept, every key below t - tau_i evicted, and
    any disagreement lies within 1e-4 * (M_i + M_t) of t; the GPU keeps
    exactly B keys per head, ascending, and its own kept set is the top-B of
    its own scores with ties to the lower slot; compacted rows are bit-exact
    copies of the input rows at the GPU's kept list, and equal the oracle's
    output wherever the kept sets agree.
Full-size workloads run in the launch configuration the benchmark times; the
oracle checks a sample of heads there (inputs copied to the host before the
pass), and properties that hold at any size are checked on every head.
"""
import os
import sys
import time
import zlib

import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri

pytestmark = pytest.mark.gpu

TOL = 2e-3      # score tolerance relative to the per-key bound M
TIGHT = 1e-4    # disagreement band around the threshold, relative to M


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(tri.LIBRARY):
        pytest.fail("libtri.so is not built")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.load()


# ------------------------------------------------------------------ helpers

def ctx_for(cache):
    sp, cal = cache.spec, cache.calib
    return tri.tri_calibrate_load(sp.n_layers, sp.n_kv_heads, sp.head_dim, cal.qc_re, cal.qc_im,
                                  cal.q_mean_norm, cal.q_mrl, cal.offsets,
                                  rope_theta=cal.rope_theta, device=0)


def seqs_for(cache):
    return [tri.Seq(cache.k[s], cache.v[s], cache.pos[s], cache.lens[s], cache.p_now[s])
            for s in range(cache.spec.n_seq)]


def score_offsets(cache):
    H = cache.spec.heads
    offs, o = [], 0
    for n in cache.lens:
        offs.append(o)
        o += H * n
    return offs, o


def head_inputs(cache, s, l, h):
    n = cache.lens[s]
    K = cache.k[s][l, h, :n].float().cpu().numpy()
    V = cache.v[s][l, h, :n].cpu()
    P = cache.pos[s][l, h, :n].cpu().numpy()
    return K, V, P


def oracle_scores(orc, cache, s, l, h, K, P):
    sp, cal = cache.spec, cache.calib
    om = orc.omega(sp.head_dim, sp.rope_theta)
    args = (cal.qc_re[l, h], cal.qc_im[l, h], cal.q_mean_norm[l, h], cal.q_mrl[l, h])
    _, _, score = orc.score_head(K, P, cache.p_now[s], om, cal.offsets, *args)
    M = orc.bound_head(K, om, cal.offsets, *args)
    return score, M


def bits(t):
    """Integer view of a tensor's elements (bit-exact comparisons)."""
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])


def check_scores(s_gpu, s_ref, M, what):
    err = np.abs(s_gpu.astype(np.float64) - s_ref) / M
    say("  %s: max |ds|/M = %.3g over %d keys" % (what, err.max(), len(err)))
    assert np.all(np.isfinite(s_gpu))
    assert err.max() <= TOL
    return err.max()


def check_kept_vs_oracle(orc, s_ref, M, P, kept_gpu, B, window, what):
    n = len(s_ref)
    kept_ref = orc.select_head(s_ref, P, B, window)
    order = np.lexsort((P, -s_ref))
    ti = order[B - 1]
    t, Mt = s_ref[ti], M[ti]
    sel = np.zeros(n, bool)
    sel[kept_gpu] = True
    assert sel.sum() == B
    tau = TOL * (M + Mt)
    assert sel[s_ref > t + tau].all(), what + ": a clearly kept key was evicted"
    assert not sel[s_ref < t - tau].any(), what + ": a clearly evicted key was kept"
    ref = np.zeros(n, bool)
    ref[kept_ref] = True
    dis = np.nonzero(ref != sel)[0]
    if len(dis):
        assert np.all(np.abs(s_ref[dis] - t) <= TIGHT * (M[dis] + Mt)), what
    say("  %s: kept-set disagreements with the oracle: %d of %d" % (what, len(dis), B))
    return kept_ref, len(dis)


def check_topb_property(scores_hn, kept_hb, n):
    """GPU-internal: per head, kept = top-B of the GPU's own scores, equal
    scores to the lower slot, strictly ascending slots in [0, n)."""
    H, B = kept_hb.shape
    kept_l = kept_hb.long()
    assert bool((kept_l[:, 1:] > kept_l[:, :-1]).all())
    assert int(kept_l.min()) >= 0 and int(kept_l.max()) < n
    mask = torch.zeros((H, n), dtype=torch.bool, device=scores_hn.device)
    mask.scatter_(1, kept_l, True)
    assert bool((mask.sum(1) == B).all())
    s = scores_hn
    inf = torch.tensor(float("inf"), device=s.device)
    kmin = torch.where(mask, s, inf).min(1).values
    emax = torch.where(~mask, s, -inf).max(1).values
    assert bool((kmin >= emax).all()), "a kept key scores below an evicted one"
    tie = kmin == emax
    if bool(tie.any()):
        slots = torch.arange(n, device=s.device)[None, :].expand(H, n)
        at_t = s == kmin[:, None]
        big = torch.tensor(n, device=s.device)
        last_kept = torch.where(mask & at_t, slots, -1).max(1).values
        first_ev = torch.where(~mask & at_t, slots, big).min(1).values
        assert bool((last_kept[tie] < first_ev[tie]).all()), "tie not broken by the lower slot"


# ------------------------------------------------------------------- scores

@pytest.mark.parametrize("name", ["toy", "llama8b_small", "f32_d128", "bf16_d64"])
def test_score_parity_all_heads(orc, name):
    if name == "toy":
        spec = synth.workload("toy")
    elif name == "llama8b_small":
        spec = synth.workload("llama8b").replace(n_layers=2, lengths=(3001,))
    elif name == "f32_d128":
        spec = synth.workload("llama8b").replace(n_layers=1, n_kv_heads=3, lengths=(2500,), dtype="f32")
    else:
        spec = synth.workload("toy").replace(dtype="bf16", lengths=(1500,), n_kv_heads=3)
    say("score parity", name, spec.lengths)
    cache = synth.make_cache(spec, "cuda", seed=1)
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    _, total = score_offsets(cache)
    scores = torch.full((total,), float("nan"), device="cuda")
    tri.tri_score(ctx, seqs, scores)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy().reshape(spec.n_layers, spec.n_kv_heads, -1)
    for l in range(spec.n_layers):
        for h in range(spec.n_kv_heads):
            K, _, P = head_inputs(cache, 0, l, h)
            s_ref, M = oracle_scores(orc, cache, 0, l, h, K, P)
            check_scores(sg[l, h], s_ref, M, "%s l%d h%d" % (name, l, h))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("n", [1, 77, 129, 257, 300])
def test_score_parity_short_and_ragged_heads(orc, dtype, d, n):
    """Heads shorter than one workgroup's tile and tails one row past a tile
    (tiles are 128 rows, 256 for bf16 with head_dim 64)."""
    spec = synth.workload("toy").replace(dtype=dtype, head_dim=d, lengths=(n,), n_kv_heads=2)
    say("score parity short", dtype, d, n)
    cache = synth.make_cache(spec, "cuda", seed=n)
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    _, total = score_offsets(cache)
    scores = torch.full((total,), float("nan"), device="cuda")
    tri.tri_score(ctx, seqs, scores)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy().reshape(spec.n_layers, spec.n_kv_heads, -1)
    for l in range(spec.n_layers):
        for h in range(spec.n_kv_heads):
            K, _, P = head_inputs(cache, 0, l, h)
            s_ref, M = oracle_scores(orc, cache, 0, l, h, K, P)
            check_scores(sg[l, h], s_ref, M, "%s d%d n%d l%d h%d" % (dtype, d, n, l, h))


def test_score_special_tables(orc):
    """q-centre 0 (norm term only), R = 1 (trig term only), explicit
    frequencies, non-identity positions and p_now well past the newest key."""
    spec = synth.workload("llama8b").replace(n_layers=1, n_kv_heads=2, lengths=(1300,))
    pos = [synth.pruned_positions(5, 1300, start=100)]
    cache = synth.make_cache(spec, "cuda", seed=2, positions=pos, p_now=[int(pos[0][-1]) + 77])
    cal = cache.calib
    cal.qc_re[0, 0] = 0.0
    cal.qc_im[0, 0] = 0.0
    cal.q_mrl[0, 1] = 1.0
    ctx = ctx_for(cache)
    scores = torch.empty(2 * 1300, device="cuda")
    tri.tri_score(ctx, seqs_for(cache), scores)
    sg = scores.cpu().numpy().reshape(2, 1300)
    for h in range(2):
        K, _, P = head_inputs(cache, 0, 0, h)
        s_ref, M = oracle_scores(orc, cache, 0, 0, h, K, P)
        check_scores(sg[h], s_ref, M, "special h%d" % h)
    inv = orc.omega(128, spec.rope_theta) * 0.5
    ctx2 = tri.tri_calibrate_load(1, 2, 128, cal.qc_re, cal.qc_im, cal.q_mean_norm, cal.q_mrl,
                                  cal.offsets, inv_freq=inv, device=0)
    tri.tri_score(ctx2, seqs_for(cache), scores)
    sg = scores.cpu().numpy().reshape(2, 1300)
    K, _, P = head_inputs(cache, 0, 0, 1)
    args = (cal.qc_re[0, 1], cal.qc_im[0, 1], cal.q_mean_norm[0, 1], cal.q_mrl[0, 1])
    _, _, s_ref = orc.score_head(K, P, cache.p_now[0], inv, cal.offsets, *args)
    M = orc.bound_head(K, inv, cal.offsets, *args)
    check_scores(sg[1], s_ref, M, "explicit inv_freq")


# ------------------------------------------------------------------- select

SELECT_CASES = [
    # kind, n, budget
    ("normal", 1000, 100), ("normal", 4097, 2048), ("ties", 3000, 700), ("allequal", 2500, 300),
    ("special", 5000, 1234), ("dups", 8192, 2048), ("ulp", 32768, 4096), ("normal", 36864, 4096),
    ("ties", 36865, 5000), ("special", 70001, 8192), ("ulp", 131072, 8192), ("normal", 300, 299),
    ("normal", 129, 1), ("straddle", 32768, 4096), ("straddle", 20000, 2048),
    ("outlier", 32768, 4096), ("outlier", 7000, 3500), ("narrow", 32768, 4096), ("narrow", 9000, 100),
    ("straddle", 131072, 8192), ("outlier", 36000, 1000),
    # positive keys whose live range runs past 2^32 - 1, with padding slots
    ("wide", 5000, 1234), ("wide", 20000, 2048), ("wide", 32768, 4096),
]


@pytest.mark.parametrize("kind,n,B", SELECT_CASES)
def test_select_bit_exact_on_synthetic_scores(orc, kind, n, B):
    H = 3
    say("select", kind, n, B)
    sc = synth.make_scores(kind, H, n, seed=n)
    pos = np.arange(n)
    k_dummy = torch.zeros((1, H, n, 64), dtype=torch.float32, device="cuda")
    ctx = tri.tri_calibrate_load(1, H, 64, np.zeros((1, H, 32)), np.zeros((1, H, 32)),
                                 np.ones((1, H, 32)), np.ones((1, H, 32)), [1], device=0)
    seq = tri.Seq(k_dummy, None, None, n, n - 1)
    kept = torch.full((H * B,), -7, dtype=torch.int32, device="cuda")
    tri.tri_select_topb(ctx, [seq], torch.from_numpy(sc.reshape(-1)).cuda(), B, 0, kept)
    kg = kept.cpu().numpy().reshape(H, B)
    for h in range(H):
        ref = orc.select_head(sc[h].astype(np.float64), pos, B, 0)
        np.testing.assert_array_equal(kg[h], ref)


def test_select_skips_heads_that_do_not_fire():
    H, n = 2, 1000
    ctx = tri.tri_calibrate_load(1, H, 64, np.zeros((1, H, 32)), np.zeros((1, H, 32)),
                                 np.ones((1, H, 32)), np.ones((1, H, 32)), [1], device=0)
    k = torch.zeros((1, H, n, 64), device="cuda")
    kept = torch.full((H * 900,), -7, dtype=torch.int32, device="cuda")
    sc = torch.randn(H * n, device="cuda")
    tri.tri_select_topb(ctx, [tri.Seq(k, None, None, n, n - 1)], sc, 900, 100, kept)
    torch.cuda.synchronize()
    assert bool((kept == -7).all())


# ------------------------------------------------------------------ compact

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("kind", ["random", "all_but_first", "every8", "last", "prefix", "blocks"])
def test_compact_bit_exact_on_synthetic_kept_lists(orc, dtype, d, kind):
    L, H, n, B = 2, 3, 5000, 1777
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(zlib.crc32(repr((kind, dtype, d)).encode()))
    K = torch.randn((L, H, n + 11, d), generator=g, device="cuda").to(tdt)
    V = torch.randn((L, H, n + 11, d), generator=g, device="cuda").to(tdt)
    P = torch.arange(n + 11, dtype=torch.int32, device="cuda").repeat(L, H, 1) * 3 + 5
    K0, V0, P0 = K.cpu(), V.cpu(), P.cpu()
    kept_np = synth.make_kept(kind, L * H, n, B, seed=d).reshape(L, H, B)
    kept = torch.from_numpy(kept_np).cuda().reshape(-1)
    ctx = tri.tri_calibrate_load(L, H, d, np.zeros((L, H, d // 2)), np.zeros((L, H, d // 2)),
                                 np.ones((L, H, d // 2)), np.ones((L, H, d // 2)), [1], device=0)
    seq = tri.Seq(K, V, P, n, n - 1)
    tri.tri_compact_kv(ctx, [seq], kept, B, 0)
    torch.cuda.synchronize()
    assert seq.len == B
    Kc, Vc, Pc = K.cpu(), V.cpu(), P.cpu()
    as_bytes = lambda t: t.contiguous().view(torch.uint8).numpy() if t.dtype != torch.int32 else t.numpy()
    for l in range(L):
        for h in range(H):
            kk = kept_np[l, h]
            np.testing.assert_array_equal(as_bytes(Kc[l, h, :B]), orc.gather_rows(kk, as_bytes(K0[l, h, :n])))
            np.testing.assert_array_equal(as_bytes(Vc[l, h, :B]), orc.gather_rows(kk, as_bytes(V0[l, h, :n])))
            np.testing.assert_array_equal(Pc[l, h, :B].numpy(), orc.gather_rows(kk, P0[l, h, :n].numpy()))


# -------------------------------------------------------------- fused pass

def _fused(orc, spec, seed, sample, full_compaction_check=True, positions=None, p_now=None):
    """Runs one prune step on the GPU as the benchmark does and checks it."""
    t0 = time.time()
    say("fused %s: generating %d keys on the GPU" % (spec.name, spec.keys))
    cache = synth.make_cache(spec, "cuda", seed=seed, positions=positions, p_now=p_now)
    torch.cuda.synchronize()
    say("  generated in %.1fs" % (time.time() - t0))
    H, B, W = spec.heads, spec.budget, spec.window
    ins = {}
    for (s, l, h) in sample:
        ins[(s, l, h)] = head_inputs(cache, s, l, h)
    pristine = None
    if full_compaction_check:
        pristine = [(cache.k[s].clone(), cache.v[s].clone(), cache.pos[s].clone())
                    for s in range(spec.n_seq)]
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    offs, total = score_offsets(cache)
    scores = torch.empty(total, device="cuda")
    kept = torch.full((spec.n_seq * H * B,), -1, dtype=torch.int32, device="cuda")
    fired = [tri.fires(q, B, W) for q in seqs]
    t1 = time.time()
    tri.prune_step(ctx, seqs, B, W, scores, kept)
    torch.cuda.synchronize()
    say("  prune step done (%.3fs incl. launch)" % (time.time() - t1))
    kept3 = kept.view(spec.n_seq, H, B)
    for s in range(spec.n_seq):
        n = cache.lens[s]
        if not fired[s]:
            assert seqs[s].len == n
            continue
        assert seqs[s].len == B
        sc = scores[offs[s]:offs[s] + H * n].view(H, n)
        check_topb_property(sc, kept3[s], n)
        if pristine is not None:
            K0, V0, P0 = pristine[s]
            idx = kept3[s].long().view(spec.n_layers, spec.n_kv_heads, B)
            for X, X0 in ((cache.k[s], K0), (cache.v[s], V0)):
                g = torch.gather(X0, 2, idx[..., None].expand(-1, -1, -1, X0.shape[-1]))
                assert torch.equal(bits(X[:, :, :B]), bits(g))
                del g
            assert torch.equal(cache.pos[s][:, :, :B], torch.gather(P0, 2, idx.int().long()).int())
        elif positions is None:
            # positions were 0..n-1, so compacted positions equal the kept slots
            assert torch.equal(cache.pos[s][:, :, :B].reshape(H, B), kept3[s])
    worst = 0.0
    for (s, l, h), (K, V, P) in ins.items():
        n = cache.lens[s]
        hi = l * spec.n_kv_heads + h
        s_ref, M = oracle_scores(orc, cache, s, l, h, K, P)
        sg = scores[offs[s] + hi * n: offs[s] + (hi + 1) * n].cpu().numpy()
        worst = max(worst, check_scores(sg, s_ref, M, "s%d l%d h%d" % (s, l, h)))
        if not fired[s]:
            continue
        kg = kept3[s, hi].cpu().numpy()
        kept_ref, ndis = check_kept_vs_oracle(orc, s_ref, M, P, kg, B, W, "s%d l%d h%d" % (s, l, h))
        Kc = cache.k[s][l, h, :B].cpu()
        Vc = cache.v[s][l, h, :B].cpu()
        Pc = cache.pos[s][l, h, :B].cpu().numpy()
        Kin = torch.from_numpy(K).to(cache.k[s].dtype)      # exact: K came from this dtype
        kgl = torch.from_numpy(kg).long()
        np.testing.assert_array_equal(Pc, P[kg])
        assert torch.equal(bits(Kc), bits(Kin[kgl]))
        assert torch.equal(bits(Vc), bits(V[kgl]))
        if ndis == 0:
            np.testing.assert_array_equal(Pc, orc.gather_rows(kept_ref, P))
            np.testing.assert_array_equal(bits(Kc).numpy(), orc.gather_rows(kept_ref, bits(Kin).numpy()))
            np.testing.assert_array_equal(bits(Vc).numpy(), orc.gather_rows(kept_ref, bits(V).numpy()))
    say("  %s: worst |ds|/M on sampled heads %.3g; total %.1fs" % (spec.name, worst, time.time() - t0))
    del cache, pristine, scores, kept
    torch.cuda.empty_cache()


def test_fused_toy_all_heads(orc):
    spec = synth.workload("toy")
    _fused(orc, spec, 0, [(0, 0, 0), (0, 0, 1)])


def test_fused_toy_pruned_positions(orc):
    """Positions with gaps (a cache pruned before): ties and the oracle's
    position order still agree with the GPU's slot order."""
    spec = synth.workload("toy").replace(lengths=(777,))
    pos = [synth.pruned_positions(3, 777, start=40)]
    _fused(orc, spec, 4, [(0, 0, 0), (0, 0, 1)], positions=pos, p_now=[int(pos[0][-1]) + 128])


def test_fused_llama8b_full(orc):
    spec = synth.workload("llama8b")
    _fused(orc, spec, 0, [(0, 0, 0), (0, 5, 3), (0, 17, 7), (0, 31, 2)])


def test_fused_qwen3_32k_full(orc):
    spec = synth.workload("qwen3_32k")
    _fused(orc, spec, 0, [(0, 0, 0), (0, 11, 4), (0, 35, 7)])


def test_fused_wide_near_ties_full(orc):
    spec = synth.workload("wide")
    _fused(orc, spec, 0, [(0, 0, 0), (0, 63, 7)])


def test_fused_batched_full(orc):
    spec = synth.workload("batched")
    lens = spec.lengths
    s_max = int(np.argmax(lens))
    s_min = int(np.argmin(lens))
    _fused(orc, spec, 0, [(s_min, 0, 0), (s_max, 31, 7), (7, 13, 2)], full_compaction_check=False)


def test_fused_mixed_firing_batch(orc):
    """Ragged batch where some sequences do not fire (len <= B + window)."""
    spec = synth.workload("llama8b").replace(name="mixed", n_layers=2, lengths=(2176, 2177, 5000, 100, 9000))
    _fused(orc, spec, 9, [(1, 0, 0), (2, 1, 7), (4, 0, 3), (0, 1, 1)])


def test_exact_duplicate_rows_keep_the_lower_slot(orc):
    """Bit-identical stored rows score bit-identically on the GPU.  With every
    row stored twice (slots i and i + 2000) and an odd budget 2m - 1, the top
    m - 1 pairs are kept whole and of the m-th pair only the lower slot."""
    B = 999
    spec = synth.workload("llama8b").replace(name="dups", n_layers=1, n_kv_heads=2, lengths=(4000,),
                                             budget=B)
    cache = synth.make_cache(spec, "cuda", seed=11)
    K = cache.k[0]
    K[:, :, 2000:4000] = K[:, :, 0:2000].clone()
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    scores = torch.empty(2 * 4000, device="cuda")
    kept = torch.empty(2 * B, dtype=torch.int32, device="cuda")
    tri.tri_score(ctx, seqs, scores)
    tri.tri_select_topb(ctx, seqs, scores, B, 128, kept)
    torch.cuda.synchronize()
    sc = scores.view(2, 4000)
    assert torch.equal(bits(sc[:, :2000]), bits(sc[:, 2000:]))
    check_topb_property(sc, kept.view(2, B), 4000)
    for h in range(2):
        # the definition on the GPU's own scores: stable sort by score, descending
        order = torch.sort(-sc[h], stable=True).indices[:B]
        assert torch.equal(kept.view(2, B)[h], torch.sort(order).values.int())
        kk = kept.view(2, B)[h].cpu().numpy()
        lo, hi = kk[kk < 2000], kk[kk >= 2000] - 2000
        # a kept copy at i + 2000 implies the kept copy at i; B odd splits a pair
        assert set(hi.tolist()) <= set(lo.tolist()) and len(lo) > len(hi)


def test_prune_then_append_then_prune(orc):
    """The decode-time cycle with uniform budgets: prune to B, append a window
    of 128 new keys (positions past p_now) to every head, prune again.  The
    oracle replays both prunes from the same inputs; the final K, V and
    positions are compared bit for bit."""
    L, H1, n, W, B = 2, 8, 3000, 128, 700
    spec = synth.workload("llama8b").replace(name="cycle", n_layers=L, lengths=(n, W), budget=B,
                                             window=W)
    pos_new = np.arange(n + 5, n + 5 + W)          # a gap, as if a few tokens were dropped
    cache = synth.make_cache(spec, "cuda", seed=12, positions=[np.arange(n), pos_new],
                             p_now=[n - 1, int(pos_new[-1])], caps=[n, W])
    cal = cache.calib
    om = orc.omega(spec.head_dim, spec.rope_theta)
    K, V, P = cache.k[0], cache.v[0], cache.pos[0]
    K0f, K0b, V0, P0 = K.float().cpu().numpy(), K.cpu(), V.cpu(), P.cpu().numpy()
    Kn, Vn = cache.k[1], cache.v[1]
    Knf, Knb, Vnh = Kn.float().cpu().numpy(), Kn.cpu(), Vn.cpu()
    ctx = ctx_for(cache)
    kept = torch.empty(L * H1 * B, dtype=torch.int32, device="cuda")
    seq = tri.Seq(K, V, P, n, n - 1)
    tri.prune_step(ctx, [seq], B, W, torch.empty(L * H1 * n, device="cuda"), kept)
    torch.cuda.synchronize()
    assert seq.len == B
    K[:, :, B:B + W] = Kn
    V[:, :, B:B + W] = Vn
    P[:, :, B:B + W] = torch.from_numpy(pos_new).to(torch.int32).cuda()
    seq = tri.Seq(K, V, P, B + W, int(pos_new[-1]))
    tri.prune_step(ctx, [seq], B, W - 1, torch.empty(L * H1 * (B + W), device="cuda"), kept)
    torch.cuda.synchronize()
    assert seq.len == B
    for l in range(L):
        for h in range(H1):
            args = (cal.qc_re[l, h], cal.qc_im[l, h], cal.q_mean_norm[l, h], cal.q_mrl[l, h])
            r1 = orc.prune_head(K0f[l, h], bits(V0[l, h]).numpy(), P0[l, h], n - 1, om, cal.offsets,
                                *args, B, W)
            k1 = orc.gather_rows(r1["kept"], bits(K0b[l, h]).numpy())
            f1 = K0f[l, h][r1["kept"]]
            Kin = np.concatenate([f1, Knf[l, h]])
            Kin_b = np.concatenate([k1, bits(Knb[l, h]).numpy()])
            Vin = np.concatenate([r1["V"], bits(Vnh[l, h]).numpy()])
            Pin = np.concatenate([r1["pos"], pos_new]).astype(np.int32)
            r2 = orc.prune_head(Kin, Vin, Pin, int(pos_new[-1]), om, cal.offsets, *args, B, W - 1)
            np.testing.assert_array_equal(P[l, h, :B].cpu().numpy(), r2["pos"])
            np.testing.assert_array_equal(bits(K[l, h, :B]).cpu().numpy(),
                                          orc.gather_rows(r2["kept"], Kin_b))
            np.testing.assert_array_equal(bits(V[l, h, :B]).cpu().numpy(), r2["V"])
    say("  two uniform prune cycles agree with the oracle on all %d heads" % (L * H1))
