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


def check_scores(s_gpu, s_ref, M, what, quiet=False):
    """Scores within TOL * M; NaN exactly where the oracle has NaN (keys with
    a non-finite element), and no other non-finite value."""
    nan_ref = np.isnan(s_ref)
    assert np.array_equal(np.isnan(s_gpu), nan_ref), what + ": NaN pattern differs from the oracle"
    assert np.all(np.isfinite(s_gpu[~nan_ref]))
    ok = ~nan_ref
    err = np.abs(s_gpu[ok].astype(np.float64) - s_ref[ok]) / M[ok] if ok.any() else np.zeros(1)
    worst = float(err.max()) if len(err) else 0.0
    # the plain relative error where it is well posed: keys whose score is
    # not a cancellation, |s| >= 0.1 * M (reported; implied <= 10 * TOL)
    big = ok & (np.abs(s_ref) >= 0.1 * M)
    rel = float((np.abs(s_gpu[big].astype(np.float64) - s_ref[big]) / np.abs(s_ref[big])).max()) \
        if big.any() else 0.0
    if not quiet:
        say("  %s: max |ds|/M = %.3g over %d keys (%d NaN); max |ds|/|s| = %.3g over the %d keys "
            "with |s| >= 0.1 M" % (what, worst, int(ok.sum()), int(nan_ref.sum()), rel, int(big.sum())))
    assert worst <= TOL
    return worst


def check_kept_vs_oracle(orc, s_ref, M, P, kept_gpu, B, window, what, quiet=False):
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
    if not quiet:
        say("  %s: kept-set disagreements with the oracle: %d of %d" % (what, len(dis), B))
    return kept_ref, len(dis)


def check_topb_property(scores_hn, kept_hb, n):
    """GPU-internal: per head, kept = top-B of the GPU's own scores, equal
    scores to the lower slot, strictly ascending slots in [0, n)."""
    H, B = kept_hb.shape
    kept_l = kept_hb.long()
    nan = torch.isnan(scores_hn)
    if bool(nan.any()):
        # NaN ranks below every number: a kept NaN means every number is kept
        kept_nan = torch.gather(nan, 1, kept_l).sum(1)
        assert bool(((kept_nan == 0) | ((~nan).sum(1) <= B)).all()), "a NaN score was kept"
        # the GPU writes no -inf (non-finite totals become NaN), so -inf can stand for NaN
        scores_hn = torch.where(nan, torch.tensor(float("-inf"), device=scores_hn.device), scores_hn)
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


SENTINEL = 0x7F80BEEF     # a signalling-NaN pattern the score kernel never writes


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_score_writes_its_range_at_any_alignment(orc, dtype, d):
    """Tiles follow the 128-byte lines of the score array, so the tiling
    depends on where the array starts and on the head length.  At start
    offsets across a line and head lengths around a line and a tile: every
    score is written, bit-identical to those of a line-aligned array (each
    key's arithmetic does not depend on its tile), the aligned scores meet
    the oracle, and nothing outside the array is written.  Several sequences
    in one call start their score ranges anywhere in a line too."""
    for n in (1, 31, 33, 129, 300, 513):
        spec = synth.workload("toy").replace(dtype=dtype, head_dim=d, lengths=(n,), n_kv_heads=3)
        cache = synth.make_cache(spec, "cuda", seed=n)
        ctx = ctx_for(cache)
        seqs = seqs_for(cache)
        total = spec.heads * n
        ref = None
        for off in (0, 1, 5, 16, 31):
            buf = torch.empty(32 + off + total + 64, dtype=torch.int32, device="cuda").fill_(SENTINEL)
            assert buf.data_ptr() % 128 == 0
            out = buf[32 + off:32 + off + total].view(torch.float32)
            tri.tri_score(ctx, seqs, out)
            torch.cuda.synchronize()
            assert bool((buf[:32 + off] == SENTINEL).all()), "written before the array (off %d)" % off
            assert bool((buf[32 + off + total:] == SENTINEL).all()), "written past the array (off %d)" % off
            got = buf[32 + off:32 + off + total].clone()
            assert not bool((got == SENTINEL).any()), "a score was not written (n %d, off %d)" % (n, off)
            if ref is None:
                ref = got
                sg = got.view(torch.float32).cpu().numpy().reshape(spec.n_layers, spec.n_kv_heads, n)
                for h in range(spec.n_kv_heads):
                    K, _, P = head_inputs(cache, 0, 0, h)
                    s_ref, M = oracle_scores(orc, cache, 0, 0, h, K, P)
                    check_scores(sg[0, h], s_ref, M, "%s d%d n%d h%d" % (dtype, d, n, h), quiet=True)
            else:
                assert torch.equal(got, ref), "scores depend on the array's alignment (n %d, off %d)" % (n, off)
    # several sequences: each one's range starts wherever the previous ended
    lens = (33, 1, 129, 300, 31)
    spec = synth.workload("toy").replace(dtype=dtype, head_dim=d, lengths=lens, n_kv_heads=3)
    cache = synth.make_cache(spec, "cuda", seed=7)
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    offs, total = score_offsets(cache)
    for off in (0, 7):
        buf = torch.empty(32 + off + total + 64, dtype=torch.int32, device="cuda").fill_(SENTINEL)
        tri.tri_score(ctx, seqs, buf[32 + off:32 + off + total].view(torch.float32))
        torch.cuda.synchronize()
        assert bool((buf[:32 + off] == SENTINEL).all()) and bool((buf[32 + off + total:] == SENTINEL).all())
        for s in range(len(lens)):
            one = torch.empty(spec.heads * lens[s], device="cuda")
            tri.tri_score(ctx, [seqs[s]], one)
            torch.cuda.synchronize()
            part = buf[32 + off + offs[s]:32 + off + offs[s] + spec.heads * lens[s]]
            assert torch.equal(part, bits(one)), "sequence %d of the batch (off %d)" % (s, off)
    say("  %s d%d: scores identical at every alignment" % (dtype, d))


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


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_nonfinite_keys_score_nan_and_are_evicted(orc, dtype, d):
    """Keys whose stored row holds +inf, -inf or NaN (one element, or +inf in
    both halves of a band) score NaN exactly where the oracle does, every
    other key within the score bar; the fused step then evicts every such
    key and compacts the rest bit for bit."""
    n, B, W = 700, 128, 128
    spec = synth.workload("toy").replace(name="nonfinite", dtype=dtype, head_dim=d, lengths=(n,),
                                         n_kv_heads=2, budget=B, window=W)
    say("non-finite keys", dtype, d)
    cache = synth.make_cache(spec, "cuda", seed=21)
    K = cache.k[0]
    rng = np.random.default_rng(21 + d)
    bad = {}
    for l in range(spec.n_layers):
        for h in range(spec.n_kv_heads):
            slots = rng.choice(n, 40, replace=False)
            bad[(l, h)] = np.sort(slots)
            for j, i in enumerate(slots):
                col = int(rng.integers(0, d))
                kind = j % 4
                if kind == 0:
                    K[l, h, i, col] = float("inf")
                elif kind == 1:
                    K[l, h, i, col] = float("-inf")
                elif kind == 2:
                    K[l, h, i, col] = float("nan")
                else:
                    f = col % (d // 2)
                    K[l, h, i, f] = float("inf")
                    K[l, h, i, f + d // 2] = float("inf")
    ctx = ctx_for(cache)
    seqs = seqs_for(cache)
    H = spec.heads
    ins = {(l, h): head_inputs(cache, 0, l, h) for l in range(spec.n_layers)
           for h in range(spec.n_kv_heads)}
    K0 = cache.k[0].clone()
    V0 = cache.v[0].clone()
    scores = torch.full((H * n,), 7.0, device="cuda")
    tri.tri_score(ctx, seqs, scores)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy().reshape(spec.n_layers, spec.n_kv_heads, n)
    refs = {}
    for (l, h), (Kh, Vh, P) in ins.items():
        s_ref, M = oracle_scores(orc, cache, 0, l, h, Kh, P)
        assert np.array_equal(np.nonzero(np.isnan(s_ref))[0], bad[(l, h)])
        check_scores(sg[l, h], s_ref, M, "%s d%d l%d h%d" % (dtype, d, l, h))
        refs[(l, h)] = (s_ref, M, P)
    kept = torch.empty(H * B, dtype=torch.int32, device="cuda")
    tri.prune_step(ctx, seqs, B, W, torch.empty(H * n, device="cuda"), kept)
    torch.cuda.synchronize()
    assert seqs[0].len == B
    kg = kept.view(spec.n_layers, spec.n_kv_heads, B)
    for (l, h), (s_ref, M, P) in refs.items():
        k_np = kg[l, h].cpu().numpy()
        assert not np.isin(k_np, bad[(l, h)]).any(), "a key with a non-finite element was kept"
        check_kept_vs_oracle(orc, s_ref, M, P, k_np, B, W, "%s d%d l%d h%d" % (dtype, d, l, h))
        idx = kg[l, h].long()
        assert torch.equal(bits(cache.k[0][l, h, :B]), bits(K0[l, h, idx]))
        assert torch.equal(bits(cache.v[0][l, h, :B]), bits(V0[l, h, idx]))
        assert torch.equal(cache.pos[0][l, h, :B], kg[l, h])


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
    # heads past the register-resident sizes (the sampled single-read
    # selection): its bracket, all keys equal, a sample that misses the
    # high runs, a threshold inside a dense cluster (too many candidates),
    # and the largest size it takes and one past it
    ("normal", 32769, 4096), ("allequal", 131072, 8192), ("ties", 131072, 8192),
    ("dups", 131072, 8192), ("runs_high", 131072, 8192), ("runs_high", 70001, 4096),
    ("cluster", 131072, 8192), ("special", 131072, 1), ("wide", 131072, 8192),
    ("normal", 262144, 16384), ("straddle", 262145, 1000),
    # budgets near the head length and tiny ones on long heads (the bracket
    # at the ends of the sample)
    ("normal", 40000, 39999), ("ties", 100000, 90000), ("normal", 262144, 250000),
    ("outlier", 200000, 7), ("cluster", 65536, 60000),
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

def row_fingerprints(X, w):
    """int64 [L][H][cap] fingerprint of every row of X [L][H][cap][d]: the
    sum over the row of its elements' bit patterns times fixed random weights
    (equal rows give equal fingerprints; rows that differ in any bit differ
    unless the weighted differences cancel exactly)."""
    out = torch.empty(X.shape[:3], dtype=torch.int64, device=X.device)
    for l in range(X.shape[0]):
        out[l] = (bits(X[l]).to(torch.int64) * w).sum(-1)
    return out


def _oracle_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _fused(orc, spec, seed, sample, compaction="pristine", positions=None, p_now=None):
    """Runs one prune step on the GPU as the benchmark does and checks it.

    sample      heads (s, l, h) compared with the oracle (scores, kept set,
                compacted rows), or "all" for every head of every sequence;
                the oracle runs on the host cores, one head per thread
    compaction  "pristine": a device copy of the cache checks the compacted
                K, V and positions of every head bit for bit;
                "fingerprint": per-row fingerprints of K and V taken before
                the step check every head's compacted rows (for caches with
                no room for a copy)
    """
    t0 = time.time()
    say("fused %s: generating %d keys on the GPU" % (spec.name, spec.keys))
    cache = synth.make_cache(spec, "cuda", seed=seed, positions=positions, p_now=p_now)
    torch.cuda.synchronize()
    say("  generated in %.1fs" % (time.time() - t0))
    H, B, W = spec.heads, spec.budget, spec.window
    if sample == "all":
        sample = [(s, l, h) for s in range(spec.n_seq) for l in range(spec.n_layers)
                  for h in range(spec.n_kv_heads)]
    # inputs of the oracle's heads, on the host before the pass
    by_seq = {}
    for (s, l, h) in sample:
        by_seq.setdefault(s, set()).add((l, h))
    host_in = {}
    for s, heads in by_seq.items():
        if len(heads) == H:
            host_in[s] = (cache.k[s].cpu(), bits(cache.v[s]).cpu(), cache.pos[s].cpu())
        else:
            for (l, h) in heads:
                host_in[(s, l, h)] = (cache.k[s][l, h].cpu(), bits(cache.v[s][l, h]).cpu(),
                                      cache.pos[s][l, h].cpu())
    pristine, fps = None, None
    if compaction == "pristine":
        pristine = [(cache.k[s].clone(), cache.v[s].clone(), cache.pos[s].clone())
                    for s in range(spec.n_seq)]
    else:
        g = torch.Generator(device="cuda")
        g.manual_seed(seed + 1)
        w = torch.randint(1, 1 << 31, (spec.head_dim,), generator=g, device="cuda", dtype=torch.int64)
        fps = [(row_fingerprints(cache.k[s], w), row_fingerprints(cache.v[s], w), w)
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
    heads_compacted = 0
    for s in range(spec.n_seq):
        n = cache.lens[s]
        if not fired[s]:
            assert seqs[s].len == n
            continue
        assert seqs[s].len == B
        sc = scores[offs[s]:offs[s] + H * n].view(H, n)
        check_topb_property(sc, kept3[s], n)
        idx = kept3[s].long().view(spec.n_layers, spec.n_kv_heads, B)
        if pristine is not None:
            K0, V0, P0 = pristine[s]
            for X, X0 in ((cache.k[s], K0), (cache.v[s], V0)):
                g = torch.gather(X0, 2, idx[..., None].expand(-1, -1, -1, X0.shape[-1]))
                assert torch.equal(bits(X[:, :, :B]), bits(g))
                del g
            assert torch.equal(cache.pos[s][:, :, :B], torch.gather(P0, 2, idx).int())
        else:
            fk, fv, w = fps[s]
            for X, f0 in ((cache.k[s], fk), (cache.v[s], fv)):
                f1 = row_fingerprints(X[:, :, :B], w)
                assert torch.equal(f1, torch.gather(f0, 2, idx)), "compacted rows differ from the kept rows"
            if positions is None:
                # positions were 0..n-1, so compacted positions equal the kept slots
                assert torch.equal(cache.pos[s][:, :, :B].reshape(H, B), kept3[s])
        heads_compacted += H
    say("  compaction checked bit for bit on %d heads (%s)" % (heads_compacted, compaction))

    # oracle checks, one head per host thread
    sc_host = {s: scores[offs[s]:offs[s] + H * cache.lens[s]].view(H, -1).cpu().numpy()
               for s in by_seq}
    kept_host = kept3.cpu().numpy()
    out_host = {s: (cache.k[s][:, :, :B].cpu(), bits(cache.v[s][:, :, :B]).cpu(),
                    cache.pos[s][:, :, :B].cpu().numpy()) for s in by_seq if fired[s]}

    def one(key):
        s, l, h = key
        n = cache.lens[s]
        if s in host_in:
            Kx, Vx, Px = (x[l, h] for x in host_in[s])
        else:
            Kx, Vx, Px = host_in[key]
        Kb, V, P = Kx[:n], Vx[:n], Px[:n].numpy()
        K = Kb.float().numpy()
        s_ref, M = oracle_scores(orc, cache, s, l, h, K, P)
        hi = l * spec.n_kv_heads + h
        worst = check_scores(sc_host[s][hi], s_ref, M, "s%d l%d h%d" % key, quiet=True)
        if not fired[s]:
            return worst, 0
        kg = kept_host[s, hi]
        kept_ref, ndis = check_kept_vs_oracle(orc, s_ref, M, P, kg, B, W, "s%d l%d h%d" % key,
                                              quiet=True)
        Kc, Vc, Pc = out_host[s]
        kgl = torch.from_numpy(kg).long()
        np.testing.assert_array_equal(Pc[l, h], P[kg])
        assert torch.equal(bits(Kc[l, h]), bits(Kb)[kgl])
        assert torch.equal(Vc[l, h], V[kgl])
        if ndis == 0:
            np.testing.assert_array_equal(Pc[l, h], orc.gather_rows(kept_ref, P))
            np.testing.assert_array_equal(bits(Kc[l, h]).numpy(), orc.gather_rows(kept_ref, bits(Kb).numpy()))
            np.testing.assert_array_equal(Vc[l, h].numpy(), orc.gather_rows(kept_ref, V.numpy()))
        return worst, ndis

    t2 = time.time()
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=_oracle_threads()) as ex:
        res = list(ex.map(one, sample))
    worst = max(r[0] for r in res)
    ndis = sum(r[1] for r in res)
    say("  %s: oracle checked %d heads (%d keys) on %d threads in %.1fs: worst |ds|/M %.3g, "
        "kept-set disagreements %d; total %.1fs"
        % (spec.name, len(sample), sum(cache.lens[s] for s, _, _ in sample), _oracle_threads(),
           time.time() - t2, worst, ndis, time.time() - t0))
    del cache, pristine, fps, scores, kept, host_in, out_host
    torch.cuda.empty_cache()
    return len(sample)


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
    """Every one of the 256 heads against the oracle."""
    spec = synth.workload("llama8b")
    assert _fused(orc, spec, 0, "all") == spec.heads


def test_fused_qwen3_32k_full(orc):
    """Every one of the 288 heads against the oracle."""
    spec = synth.workload("qwen3_32k")
    assert _fused(orc, spec, 0, "all") == spec.heads


def test_fused_wide_near_ties_full(orc):
    """One head of every layer (64 of 512) against the oracle; every head's
    compaction bit for bit."""
    spec = synth.workload("wide")
    sample = [(0, l, (5 * l) % spec.n_kv_heads) for l in range(spec.n_layers)]
    assert _fused(orc, spec, 0, sample) == spec.n_layers


def test_fused_batched_full(orc):
    """64 ragged sequences: the compaction of all 16,384 heads checked by row
    fingerprints, the top-B property on every head, sampled heads against
    the oracle."""
    spec = synth.workload("batched")
    lens = spec.lengths
    s_max = int(np.argmax(lens))
    s_min = int(np.argmin(lens))
    sample = [(s_min, 0, 0), (s_max, 31, 7), (7, 13, 2)] + [(s, s % spec.n_layers, s % spec.n_kv_heads)
                                                            for s in range(0, spec.n_seq, 8)]
    _fused(orc, spec, 0, sample, compaction="fingerprint")


def test_fused_mixed_firing_batch(orc):
    """Ragged batch where some sequences do not fire (len <= B + window)."""
    spec = synth.workload("llama8b").replace(name="mixed", n_layers=2, lengths=(2176, 2177, 5000, 100, 9000))
    _fused(orc, spec, 9, [(1, 0, 0), (2, 1, 7), (4, 0, 3), (0, 1, 1)])


def test_fused_many_sequences_every_length_class(orc):
    """70 sequences in one call: more than one launch's table of sequences
    for the batched selection (64) and compaction (32), every register-
    resident length class (up to 8192, 16384 and 32768 keys), heads longer
    than 32768 keys (selected one sequence at a time), and sequences at the
    firing boundary that do not fire."""
    B, W = 300, 128
    edge = [B + W, B + W + 1, 8192, 8193, 16384, 16385, 32768, 32769, 40000]
    rng = np.random.default_rng(31)
    lens = edge + [int(x) for x in rng.integers(B + W - 50, 33000, size=70 - len(edge))]
    spec = synth.workload("llama8b").replace(name="many", n_layers=1, n_kv_heads=2,
                                             lengths=tuple(lens), budget=B, window=W)
    sample = [(s, 0, s % 2) for s in range(0, len(lens), 3)]
    assert _fused(orc, spec, 13, sample) == len(sample)


def _random_spec(case):
    """A seeded small configuration: dtype, head_dim, layers, KV heads,
    ragged lengths (some at or below the firing boundary), budget, window,
    RoPE base, offset set and key recipe."""
    rng = np.random.default_rng(1000 + case)
    recipe = ["toy", "concentrated", "phase", "neartie"][int(rng.integers(4))]
    dtype = "bf16" if recipe == "neartie" else ["bf16", "f32"][int(rng.integers(2))]
    d = [64, 128][int(rng.integers(2))]
    budget, window = int(rng.integers(1, 1500)), int(rng.integers(0, 200))
    lengths = [int(x) for x in rng.integers(1, 5000, size=int(rng.integers(1, 4)))]
    if rng.random() < 0.4:
        lengths[int(rng.integers(len(lengths)))] = int(rng.integers(1, budget + window + 1))
    return synth.workload("toy").replace(
        name="random%d" % case, n_layers=int(rng.integers(1, 3)), n_kv_heads=int(rng.integers(1, 4)),
        head_dim=d, rope_theta=float([1e4, 5e5, 1e6][int(rng.integers(3))]), lengths=tuple(lengths),
        budget=budget, window=window, dtype=dtype, recipe=recipe,
        offsets=synth.pow2_offsets(int(rng.integers(8, 17))),
        dup_frac=0.1 if recipe == "neartie" else 0.0,
        outlier_frac=0.05 if recipe == "concentrated" else 0.0)


@pytest.mark.parametrize("case", range(24))
def test_fused_random_small_configs(orc, case):
    """Seeded random small configurations through the whole prune step, every
    head against the oracle (scores, kept set, compaction bit for bit)."""
    spec = _random_spec(case)
    say("random config", case, spec.dtype, spec.head_dim, spec.n_layers, spec.n_kv_heads,
        spec.lengths, spec.budget, spec.window, spec.recipe, spec.rope_theta)
    sample = [(s, l, h) for s in range(spec.n_seq) for l in range(spec.n_layers)
              for h in range(spec.n_kv_heads)]
    assert _fused(orc, spec, case, sample) == len(sample)


def test_degenerate_calls(orc):
    """No sequences at all; a batch with empty sequences, a one-key sequence,
    one exactly at the firing boundary (len = budget + window, does not fire)
    and one just past it (fires) beside a long one."""
    spec = synth.workload("toy")
    cache = synth.make_cache(spec, "cuda", seed=0)
    ctx = ctx_for(cache)
    empty_f = torch.empty(0, device="cuda")
    empty_i = torch.empty(0, dtype=torch.int32, device="cuda")
    tri.prune_step(ctx, [], spec.budget, spec.window, empty_f, empty_i)
    torch.cuda.synchronize()
    B, W = spec.budget, spec.window
    spec2 = spec.replace(name="degenerate", lengths=(0, 1, 700, 0, B + W, B + W + 1))
    sample = [(2, 0, 0), (2, 0, 1), (5, 0, 1), (1, 0, 0), (4, 0, 0)]
    assert _fused(orc, spec2, 17, sample) == len(sample)


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


def test_prune_steps_on_two_streams_from_two_threads():
    """The library keeps no per-call state outside its arguments: two host
    threads, each pruning its own caches on a stream of its own, give bit for
    bit the results of the same calls made one after the other on one
    stream (a single sequence and a three-sequence batch, run four times
    each, interleaved)."""
    import threading
    specs = [synth.workload("llama8b").replace(name="thread_a", n_layers=2, lengths=(3001,)),
             synth.workload("llama8b").replace(name="thread_b", n_layers=2, lengths=(2500, 9000, 2200),
                                               budget=1000)]
    caches = [synth.make_cache(sp, "cuda", seed=30 + i) for i, sp in enumerate(specs)]
    ctxs = [ctx_for(c) for c in caches]
    pristine = [[(k.clone(), v.clone(), p.clone()) for k, v, p in zip(c.k, c.v, c.pos)] for c in caches]

    def restore(i):
        for (k0, v0, p0), k, v, p in zip(pristine[i], caches[i].k, caches[i].v, caches[i].pos):
            k.copy_(k0)
            v.copy_(v0)
            p.copy_(p0)

    def step(i, stream):
        sp, c = specs[i], caches[i]
        seqs = seqs_for(c)
        _, total = score_offsets(c)
        scores = torch.empty(total, device="cuda")
        kept = torch.full((sp.n_seq * sp.heads * sp.budget,), -1, dtype=torch.int32, device="cuda")
        tri.prune_step(ctxs[i], seqs, sp.budget, sp.window, scores, kept, stream)
        return kept, [s.len for s in seqs]

    def snapshot(i, kept, lens):
        return (kept.clone(), lens, [(k.clone(), v.clone(), p.clone())
                                     for k, v, p in zip(caches[i].k, caches[i].v, caches[i].pos)])

    # one after the other on the current stream
    ref = []
    for i in range(2):
        restore(i)
        kept, lens = step(i, None)
        torch.cuda.synchronize()
        ref.append(snapshot(i, kept, lens))
    # two threads, two streams (default priority), several rounds each
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = [None, None]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            with torch.cuda.stream(streams[i]):
                for _ in range(4):
                    restore(i)
                    kept, lens = step(i, streams[i])
                streams[i].synchronize()
                out[i] = snapshot(i, kept, lens)
                streams[i].synchronize()
        except Exception as e:   # surfaced in the main thread
            errors.append(e)

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        kept_r, lens_r, rows_r = ref[i]
        kept_o, lens_o, rows_o = out[i]
        assert lens_o == lens_r
        assert torch.equal(kept_o, kept_r), specs[i].name
        for (k0, v0, p0), (k1, v1, p1) in zip(rows_r, rows_o):
            assert torch.equal(bits(k0), bits(k1)) and torch.equal(bits(v0), bits(v1))
            assert torch.equal(p0, p1)
    say("  two threads on two streams: identical to the serial calls")


@pytest.mark.parametrize("lengths", [(3001,), (2500, 9000, 2200)])
def test_prune_step_replays_from_a_hip_graph(lengths):
    """A step's calls launch kernels only (no allocation, copy or memset), so
    a caller can capture them in a HIP graph.  The graph is replayed three
    times, the cache restored eagerly and synchronized between replays, and
    every replay equals the eager step bit for bit."""
    sp = synth.workload("llama8b").replace(name="graph", n_layers=2, lengths=lengths, budget=1000)
    cache = synth.make_cache(sp, "cuda", seed=40)
    ctx = ctx_for(cache)
    pristine = [(k.clone(), v.clone(), p.clone()) for k, v, p in zip(cache.k, cache.v, cache.pos)]

    def restore():
        for (k0, v0, p0), k, v, p in zip(pristine, cache.k, cache.v, cache.pos):
            k.copy_(k0)
            v.copy_(v0)
            p.copy_(p0)

    _, total = score_offsets(cache)
    scores = torch.empty(total, device="cuda")
    kept = torch.full((sp.n_seq * sp.heads * sp.budget,), -1, dtype=torch.int32, device="cuda")
    restore()
    tri.prune_step(ctx, seqs_for(cache), sp.budget, sp.window, scores, kept)
    torch.cuda.synchronize()
    ref_kept = kept.clone()
    ref_rows = [(k.clone(), v.clone(), p.clone()) for k, v, p in zip(cache.k, cache.v, cache.pos)]

    restore()
    kept.fill_(-1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tri.prune_step(ctx, seqs_for(cache), sp.budget, sp.window, scores, kept)
    torch.cuda.synchronize()
    for r in range(3):
        restore()
        kept.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kept, ref_kept), "replay %d: kept lists" % r
        for (k0, v0, p0), k, v, p in zip(ref_rows, cache.k, cache.v, cache.pos):
            assert torch.equal(bits(k), bits(k0)) and torch.equal(bits(v), bits(v0)), "replay %d" % r
            assert torch.equal(p, p0), "replay %d: positions" % r
    say("  %d sequence(s): three graph replays equal the eager step" % sp.n_seq)


def test_rows_per_head_limit():
    """The kernels address a head's rows with 32-bit byte offsets: len *
    head_dim * 4 must stay below 2^31.  At the limit every call is an
    argument error (nothing enqueued); one key below it the score runs."""
    d = 128
    lim = (1 << 31) // (4 * d)
    ctx = tri.tri_calibrate_load(1, 1, d, np.zeros((1, 1, 64)), np.full((1, 1, 64), 0.5),
                                 np.ones((1, 1, 64)), np.full((1, 1, 64), 0.5), [1, 2], device=0)
    k = torch.zeros((1, 1, lim, d), dtype=torch.bfloat16, device="cuda")
    scores = torch.empty(lim, device="cuda")
    kept = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(tri.TriError) as e:
        tri.tri_score(ctx, [tri.Seq(k, None, None, lim, lim - 1)], scores)
    assert e.value.status == tri.TRI_E_INVAL
    with pytest.raises(tri.TriError) as e:
        tri.tri_select_topb(ctx, [tri.Seq(k, None, None, lim, lim - 1)], scores, 16, 0, kept)
    assert e.value.status == tri.TRI_E_INVAL
    tri.tri_score(ctx, [tri.Seq(k, None, None, lim - 1, lim - 2)], scores)
    torch.cuda.synchronize()
    # zero keys score zero: trig and norm both vanish
    assert float(scores[:lim - 1].abs().max()) == 0.0
    del k, scores
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [8192, 8193, 16384, 16385, 24576, 24577, 32768, 32769])
@pytest.mark.parametrize("frac", [0.0, 0.33, 1.0])
def test_select_at_the_length_class_edges(orc, n, frac):
    """Heads at and one past each register-resident length class (8, 16, 24
    and 32 keys per thread) and the single-read long-head path, with budgets
    of 1, a third and n - 1: kept lists bit-exact with the oracle, alone and
    as one sequence of a batch beside a head of another class."""
    B = max(1, min(n - 1, int(n * frac)))
    kind = ("ties", "normal", "straddle")[int(frac * 2)]
    H = 2
    sc = synth.make_scores(kind, H, n, seed=n + B)
    pos = np.arange(n)
    ctx = tri.tri_calibrate_load(1, H, 64, np.zeros((1, H, 32)), np.zeros((1, H, 32)),
                                 np.ones((1, H, 32)), np.ones((1, H, 32)), [1], device=0)
    k = torch.zeros((1, H, n, 64), dtype=torch.float32, device="cuda")
    other = 5000 if n > 9000 else 20000
    k2 = torch.zeros((1, H, other, 64), dtype=torch.float32, device="cuda")
    sc2 = synth.make_scores("normal", H, other, seed=other)
    ref = [orc.select_head(sc[h].astype(np.float64), pos, B, 0) for h in range(H)]
    # alone
    kept = torch.full((H * B,), -7, dtype=torch.int32, device="cuda")
    tri.tri_select_topb(ctx, [tri.Seq(k, None, None, n, n - 1)], torch.from_numpy(sc.reshape(-1)).cuda(),
                        B, 0, kept)
    kg = kept.cpu().numpy().reshape(H, B)
    for h in range(H):
        np.testing.assert_array_equal(kg[h], ref[h])
    # in a batch, after a sequence of another length class
    if other > B:
        both = torch.from_numpy(np.concatenate([sc2.reshape(-1), sc.reshape(-1)])).cuda()
        kept2 = torch.full((2 * H * B,), -7, dtype=torch.int32, device="cuda")
        tri.tri_select_topb(ctx, [tri.Seq(k2, None, None, other, other - 1),
                                  tri.Seq(k, None, None, n, n - 1)], both, B, 0, kept2)
        kg2 = kept2.cpu().numpy().reshape(2, H, B)
        for h in range(H):
            np.testing.assert_array_equal(kg2[1, h], ref[h])
            np.testing.assert_array_equal(
                kg2[0, h], orc.select_head(sc2[h].astype(np.float64), np.arange(other), B, 0))
