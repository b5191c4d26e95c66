"""GPU parity of the distance-preference curves (tri_distance_curve) and of
scoring with non-default future-offset sets, against the fp64 oracle.

Sources: dimensionstp.github.io TriAttention review, section 2-1 item 2,
section 2-2, section 4-3 "Future offset design", section 6 item 2;
romaanj.github.io TriAttention review, section "Method".
Bar: the curve is computed in fp64 on both sides.  With the oracle's band
frequencies passed to the context (inv_freq), both evaluate the same angles
and entries agree to 1e-9 of sum_f |E q_f| |kc_f|.  With the frequencies
derived on each side (pow on the GPU and in the C library may differ by an
ulp), the angle w_f * delta can differ by about 4 * 2^-52 * w_f * |delta|,
which is 1e-4 rad at |delta| = 2^40; the bar adds that term per band.  Scores
with other offset sets meet the score bar of the main parity tests (2e-3 * M).
"""
import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri
from test_gpu_parity import check_scores, head_inputs, say, seqs_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.load()


@pytest.mark.parametrize("name,explicit", [("gqa_toy", True), ("gqa_toy", False),
                                           ("qwen3_32k_gqa", True), ("qwen3_32k_gqa", False)])
def test_distance_curve_matches_oracle(orc, name, explicit):
    spec = synth.workload(name)
    cal = synth._model(spec, 0)[2]
    om = orc.omega(spec.head_dim, spec.rope_theta)
    ctx = tri.tri_calibrate_load(spec.n_layers, spec.n_kv_heads, spec.head_dim, cal.qc_re, cal.qc_im,
                                 cal.q_mean_norm, cal.q_mrl, cal.offsets, rope_theta=cal.rope_theta,
                                 inv_freq=om if explicit else None, device=0,
                                 n_q_heads=spec.n_q_heads)
    h = spec.head_dim // 2
    rng = np.random.default_rng(41)
    kc = rng.standard_normal((spec.heads, 2, h))
    deltas = np.array([0, 1, 2, 7, 100, 4096, 65536, 1 << 30, -5, -4096, 1 << 40], dtype=np.int64)
    curve = tri.tri_distance_curve(ctx, torch.from_numpy(kc[:, 0].copy()).cuda(),
                                   torch.from_numpy(kc[:, 1].copy()).cuda(),
                                   torch.from_numpy(deltas).cuda()).cpu().numpy()
    G = spec.group
    qre = cal.qc_re.reshape(-1, h)
    qim = cal.qc_im.reshape(-1, h)
    worst = 0.0
    heads = range(spec.heads * G) if spec.heads * G <= 64 else [0, 1, 5, 63, 500, spec.heads * G - 1]
    for qh in heads:
        kv = qh // G
        ref = orc.distance_curve(om, qre[qh], qim[qh], kc[kv, 0], kc[kv, 1], deltas)
        qk = np.hypot(qre[qh], qim[qh]) * np.hypot(kc[kv, 0], kc[kv, 1])
        tol = 1e-9 * qk.sum() + (0.0 if explicit else
                                 4 * 2.0 ** -52 * np.abs(deltas).astype(np.float64) * (om * qk).sum())
        err = np.abs(curve[qh] - ref)
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), (qh, err, tol)
    say("  %s (%s frequencies): curve max |d|/tol = %.3g" % (name, "explicit" if explicit else "derived", worst))


@pytest.mark.parametrize("kind,maxd,count", [("linear", 65536, 17), ("linear", 4096, 64),
                                             ("geometric", 4096, 0), ("geometric", 1 << 20, 0)])
def test_scores_with_other_offset_sets(orc, kind, maxd, count):
    offsets = tri.offset_set(kind, maxd, count)
    spec = synth.workload("llama8b").replace(n_layers=1, n_kv_heads=2, lengths=(3000,),
                                             offsets=tuple(int(x) for x in offsets))
    say("scores with %s offsets to %d (%d offsets)" % (kind, maxd, len(offsets)))
    cache = synth.make_cache(spec, "cuda", seed=9)
    cal = cache.calib
    ctx = tri.tri_calibrate_load(1, 2, 128, cal.qc_re, cal.qc_im, cal.q_mean_norm, cal.q_mrl,
                                 cal.offsets, rope_theta=cal.rope_theta, device=0)
    scores = torch.empty(2 * 3000, device="cuda")
    tri.tri_score(ctx, seqs_for(cache), scores)
    sg = scores.cpu().numpy().reshape(2, 3000)
    om = orc.omega(128, spec.rope_theta)
    for h in range(2):
        K, _, P = head_inputs(cache, 0, 0, h)
        args = (cal.qc_re[0, h], cal.qc_im[0, h], cal.q_mean_norm[0, h], cal.q_mrl[0, h])
        _, _, s_ref = orc.score_head(K, P, cache.p_now[0], om, cal.offsets, *args)
        M = orc.bound_head(K, om, cal.offsets, *args)
        check_scores(sg[h], s_ref, M, "%s %d h%d" % (kind, maxd, h))


@pytest.mark.parametrize("case", range(10))
def test_distance_curve_random_shapes(orc, case):
    """Seeded random shapes for the tiled curve kernel (64 distances by 64
    query heads per workgroup, bands in LDS 16 at a time): head_dim, layers,
    KV heads, G, the number of distances (tile edges included) and their
    values (negative, zero, far), with the oracle's frequencies."""
    rng = np.random.default_rng(5000 + case)
    d = [64, 128][int(rng.integers(2))]
    spec = synth.workload("gqa_toy").replace(
        name="curve_random%d" % case, n_layers=int(rng.integers(1, 4)),
        n_kv_heads=int(rng.integers(1, 9)), head_dim=d, group=int(rng.integers(1, 9)),
        rope_theta=float([1e4, 5e5, 1e6][int(rng.integers(3))]))
    n_delta = int(rng.choice([1, 63, 64, 65, 128, 129, int(rng.integers(2, 400))]))
    deltas = rng.integers(-(1 << 20), 1 << 20, size=n_delta).astype(np.int64)
    deltas[::7] = rng.integers(-(1 << 40), 1 << 40, size=deltas[::7].size)
    if n_delta > 2:
        deltas[:2] = [0, 1]
    cal = synth._model(spec, case)[2]
    om = orc.omega(d, spec.rope_theta)
    ctx = tri.tri_calibrate_load(spec.n_layers, spec.n_kv_heads, d, cal.qc_re, cal.qc_im,
                                 cal.q_mean_norm, cal.q_mrl, cal.offsets, rope_theta=cal.rope_theta,
                                 inv_freq=om, device=0, n_q_heads=spec.n_q_heads)
    h = d // 2
    kc = rng.standard_normal((spec.heads, 2, h))
    say("curve random", case, "d", d, "kv heads", spec.heads, "G", spec.group, "distances", n_delta)
    curve = tri.tri_distance_curve(ctx, torch.from_numpy(kc[:, 0].copy()).cuda(),
                                   torch.from_numpy(kc[:, 1].copy()).cuda(),
                                   torch.from_numpy(deltas).cuda()).cpu().numpy()
    G = spec.group
    qre = cal.qc_re.reshape(-1, h)
    qim = cal.qc_im.reshape(-1, h)
    assert curve.shape == (spec.heads * G, n_delta)
    for qh in range(spec.heads * G):
        kv = qh // G
        ref = orc.distance_curve(om, qre[qh], qim[qh], kc[kv, 0], kc[kv, 1], deltas)
        qk = np.hypot(qre[qh], qim[qh]) * np.hypot(kc[kv, 0], kc[kv, 1])
        assert np.all(np.abs(curve[qh] - ref) <= 1e-9 * qk.sum()), qh
