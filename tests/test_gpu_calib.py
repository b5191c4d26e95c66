"""GPU parity of the calibration statistics from pre-RoPE query samples
(tri_calibrate_stats) against the fp64 oracle, called through the C ABI.

Source: romaanj.github.io TriAttention review, section "Method";
dimensionstp.github.io TriAttention review, section 3 (calibration phase).

Bar: both sides sum the same stored samples in fp64, only in a different
order, so the centre, the mean norm and R agree to 1e-12 relative to the
mean norm of the band (n_samples * 2^-52 is below 1e-11 for every size
here).  A statistical check pins the reading R_f = |E q_f| / E|q_f| on
samples of known concentration, and a loaded context built from the GPU's
statistics scores a cache as the oracle does from its own statistics.
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


def _stats_vs_oracle(orc, q, heads):
    out = [t.cpu().numpy() for t in tri.tri_calibrate_stats(q)]
    torch.cuda.synchronize()
    qh = q.float().cpu().numpy()
    worst = 0.0
    for h in heads:
        ref = orc.calib_stats(qh[:, h, :])
        scale = np.maximum(ref[2], 1e-300)
        for got, r in zip(out, ref):
            err = np.abs(got[h] - r)
            worst = max(worst, float((err / scale).max()))
        assert np.all(np.abs(out[3][h] - ref[3]) <= 1e-12)
    assert worst <= 1e-12
    return out, worst


@pytest.mark.parametrize("dtype,d,n,H", [("bf16", 128, 20001, 6), ("f32", 64, 3000, 5), ("bf16", 64, 777, 3),
                                         ("f32", 128, 1, 2), ("bf16", 128, 33, 4)])
def test_calib_stats_match_oracle(orc, dtype, d, n, H):
    say("calibration statistics", dtype, d, n, H)
    q, _, _ = synth.query_samples(H, d, n, seed=n, dtype=dtype, device="cuda")
    _, worst = _stats_vs_oracle(orc, q, range(H))
    say("  max relative difference %.3g" % worst)


def test_calib_stats_recover_known_concentration_and_are_deterministic():
    q, R_true, centres = synth.query_samples(8, 128, 120_000, seed=3, dtype="f32", device="cuda",
                                             constant_norm=True)
    a = tri.tri_calibrate_stats(q)
    b = tri.tri_calibrate_stats(q)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    R = a[3].cpu().numpy()
    say("  |R - R_true| max %.4f" % np.abs(R - R_true).max())
    assert np.abs(R - R_true).max() < 0.012
    h = 64
    ang = np.angle((a[0].cpu().numpy() + 1j * a[1].cpu().numpy())
                   * np.exp(-1j * np.angle(centres[:, :h] + 1j * centres[:, h:])))
    assert np.abs(ang[R_true > 0.5]).max() < 0.02


def test_calibrated_context_scores_like_the_oracle(orc):
    """Statistics from samples -> tri_calibrate_load -> tri_score, against the
    oracle scoring with its own statistics of the same samples."""
    spec = synth.workload("llama8b").replace(n_layers=1, n_kv_heads=2, lengths=(2000,))
    cache = synth.make_cache(spec, "cuda", seed=7)
    q, _, _ = synth.query_samples(2, 128, 5000, seed=8, dtype="bf16", device="cuda")
    st = [t.cpu().numpy().reshape(1, 2, 64) for t in tri.tri_calibrate_stats(q)]
    ctx = tri.tri_calibrate_load(1, 2, 128, *st, spec.offsets, rope_theta=spec.rope_theta, device=0)
    scores = torch.empty(2 * 2000, device="cuda")
    tri.tri_score(ctx, seqs_for(cache), scores)
    sg = scores.cpu().numpy().reshape(2, 2000)
    qh = q.float().cpu().numpy()
    om = orc.omega(128, spec.rope_theta)
    for h in range(2):
        ref_stats = orc.calib_stats(qh[:, h, :])
        K, _, P = head_inputs(cache, 0, 0, h)
        _, _, s_ref = orc.score_head(K, P, cache.p_now[0], om, np.array(spec.offsets), *ref_stats)
        M = orc.bound_head(K, om, np.array(spec.offsets), *ref_stats)
        check_scores(sg[h], s_ref, M, "calibrated from samples h%d" % h)


@pytest.mark.parametrize("case", range(10))
def test_calib_stats_random_shapes(orc, case):
    """Seeded random sample counts, query heads, head_dim and dtype."""
    rng = np.random.default_rng(6000 + case)
    dtype, d = ["bf16", "f32"][int(rng.integers(2))], [64, 128][int(rng.integers(2))]
    n, H = int(rng.integers(1, 6000)), int(rng.integers(1, 20))
    say("calibration statistics, random", case, dtype, d, n, H)
    q, _, _ = synth.query_samples(H, d, n, seed=6000 + case, dtype=dtype, device="cuda")
    _stats_vs_oracle(orc, q, range(H))


def test_context_from_a_saved_table_scores_identically(tmp_path):
    """A calibration table written to disk and read back gives a context whose
    scores equal, bit for bit, those of the context loaded from the arrays."""
    spec = synth.workload("llama8b").replace(n_layers=2, n_kv_heads=2, lengths=(3000,))
    cache = synth.make_cache(spec, "cuda", seed=11)
    c = cache.calib
    ctx_a = tri.tri_calibrate_load(2, 2, 128, c.qc_re, c.qc_im, c.q_mean_norm, c.q_mrl, c.offsets,
                                   rope_theta=c.rope_theta, device=0)
    path = tmp_path / "calib.npz"
    tri.save_calibration(path, c.qc_re, c.qc_im, c.q_mean_norm, c.q_mrl, c.offsets, n_kv_heads=2,
                         head_dim=128, rope_theta=c.rope_theta)
    ctx_b = tri.tri_calibrate_load(**tri.load_calibration(path), device=0)
    n = 2 * 2 * 3000
    sa = torch.empty(n, device="cuda")
    sb = torch.empty(n, device="cuda")
    tri.tri_score(ctx_a, seqs_for(cache), sa)
    tri.tri_score(ctx_b, seqs_for(cache), sb)
    torch.cuda.synchronize()
    say("saved calibration table: %d scores compared" % n)
    assert torch.equal(sa, sb)
