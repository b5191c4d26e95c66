"""Pins of the fp64 oracle to things other than itself.

Every check here is independent of the oracle's own code: brute-force real
RoPE dot products built from dense rotation matrices, the pages' polar
per-band form |q||k|cos(w*dist + phi), closed-form special cases, hand-worked
fixtures under tests/golden/, library sorts and brute-force subset
enumeration.  Each is chosen so that a plausible mistake in the oracle
(a dropped term, a flipped sign or conjugate, interleaved instead of
half-split pairing, swapped query and key, a wrong tie-break) fails at least
one of them.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
# Independent re-statements used only as pins: real dense rotation matrices
# in the rotate-half layout (band f = dims f and f + d/2).

def omega_np(d, theta):
    return np.array([theta ** (-2.0 * f / d) for f in range(d // 2)])


def rope_matrix(d, p, om):
    R = np.zeros((d, d))
    h = d // 2
    for f in range(h):
        c, s = math.cos(om[f] * p), math.sin(om[f] * p)
        R[f, f], R[f, f + h] = c, -s
        R[f + h, f], R[f + h, f + h] = s, c
    return R


def qvec(qc_re, qc_im):
    return np.concatenate([qc_re, qc_im])


def random_head(rng, d, n, pmax=5000):
    h = d // 2
    qc_re, qc_im = rng.standard_normal(h), rng.standard_normal(h)
    m = np.hypot(qc_re, qc_im) * (1 + rng.uniform(0, 0.5, h))
    R = np.hypot(qc_re, qc_im) / m
    pos = np.sort(rng.choice(pmax, size=n, replace=False)).astype(np.int64)
    K = rng.standard_normal((n, d))
    return qc_re, qc_im, m, R, pos, K


# ------------------------------------------------------- frequencies / RoPE

def test_omega_matches_standard_rope(oracle_lib):
    for d, th in [(64, 1e4), (128, 5e5), (128, 1e6), (8, 10.0)]:
        np.testing.assert_allclose(oracle_lib.omega(d, th), omega_np(d, th), rtol=1e-15, atol=0)
        assert oracle_lib.omega(d, th)[0] == 1.0


def _library_rope(d, theta):
    """The rotary embedding of a widely used model library (the Llama
    rotary embedding of `transformers`): its band frequencies and a function
    that rotates rows [n, d] to the given positions.  The library computes
    the angles in fp32."""
    pytest.importorskip("transformers")
    import torch
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    cfg = LlamaConfig(hidden_size=2 * d, num_attention_heads=2, num_key_value_heads=2, head_dim=d,
                      rope_theta=theta)
    emb = LlamaRotaryEmbedding(cfg)

    def rotate(x, positions):
        t = torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None]
        cos, sin = emb(t, torch.as_tensor(np.asarray(positions), dtype=torch.long)[None])
        out, _ = apply_rotary_pos_emb(t, t, cos, sin)
        return out[0, 0].numpy()

    return emb.inv_freq.double().numpy(), rotate


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 5e5), (128, 1e6)])
def test_omega_and_bands_match_a_model_library(oracle_lib, d, theta):
    """Readings A1 (w_f = theta^(-2f/d)) and A2 (band f = dims f and f + d/2,
    turned by +w_f * p) against the RoPE of a model library instead of a
    restatement: the oracle's frequencies equal the library's (to its fp32),
    and the oracle's trig term of keys the library rotated to their
    positions equals the mean over the offsets of the dot products with the
    query centre the library rotated to p_now + delta."""
    lib_om, rotate = _library_rope(d, theta)
    om = oracle_lib.omega(d, theta)
    np.testing.assert_allclose(om, lib_om, rtol=2e-7, atol=0)
    rng = np.random.default_rng(d)
    n = 40
    k = rng.standard_normal((n, d))
    pos = np.sort(rng.choice(150, size=n, replace=False)).astype(np.int64)
    K = rotate(k, pos)                              # stored post-RoPE keys
    qc_re, qc_im = rng.standard_normal(d // 2), rng.standard_normal(d // 2)
    q = np.concatenate([qc_re, qc_im])
    offsets = np.array([1, 2, 4, 8], dtype=np.int64)
    p_now = int(pos[-1]) + 3
    ones = np.ones(d // 2)
    trig, _, _ = oracle_lib.score_head(K, pos, p_now, om, offsets, qc_re, qc_im,
                                       np.hypot(qc_re, qc_im), ones)
    lib = np.mean([K @ rotate(q[None], [p_now + int(t)])[0] for t in offsets], axis=0)
    scale = np.abs(q).sum() * np.abs(k).sum(axis=1)
    assert np.all(np.abs(trig - lib) <= 1e-6 * scale), np.max(np.abs(trig - lib) / scale)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_unrotate_inverts_a_dense_rotation(oracle_lib, d):
    rng = np.random.default_rng(d)
    om = omega_np(d, 1e4)
    for p in [0, 1, 37, 4095, 131071]:
        k = rng.standard_normal(d)
        K = rope_matrix(d, p, om) @ k
        z = oracle_lib.unrotate(K, p, om)
        np.testing.assert_allclose(z.real, k[: d // 2], atol=1e-12)
        np.testing.assert_allclose(z.imag, k[d // 2:], atol=1e-12)


def test_unrotate_composes_and_preserves_band_norms(oracle_lib):
    rng = np.random.default_rng(1)
    d = 16
    om = omega_np(d, 100.0)
    K = rng.standard_normal(d)
    a = oracle_lib.unrotate(K, 7, om)
    b = oracle_lib.unrotate(rope_matrix(d, -3, om) @ K, 4, om)   # rot(-3) then unrotate(4)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(np.abs(a), np.hypot(K[:8], K[8:]), rtol=1e-14)


# ------------------------------------------------------------ trig series

@pytest.mark.parametrize("d,n,theta", [(8, 40, 10.0), (64, 64, 1e4), (128, 24, 5e5)])
def test_trig_equals_bruteforce_rope_dot_products(oracle_lib, d, n, theta):
    """For every offset, the real dot product of the RoPE-rotated query centre
    (at p_now + delta) with the stored key equals the per-band series; the
    oracle's trig term is their mean."""
    rng = np.random.default_rng(d + n)
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, n, pmax=60000)
    om = omega_np(d, theta)
    offsets = np.array([1, 2, 4, 8, 16, 1024, 65536], dtype=np.int64)
    p_now = int(pos[-1]) + 3
    trig, norm, score = oracle_lib.score_head(K, pos, p_now, om, offsets, qc_re, qc_im, m, R)
    q = qvec(qc_re, qc_im)
    brute = np.zeros(n)
    for delta in offsets:
        qrot = rope_matrix(d, p_now + int(delta), om) @ q
        brute += K @ qrot
    brute /= len(offsets)
    scale = np.abs(q).sum() * np.abs(K).sum(axis=1)
    assert np.all(np.abs(trig - brute) <= 1e-11 * scale)


def test_trig_on_toy_workload_equals_bruteforce(oracle_lib):
    spec = synth.workload("toy")
    c = synth.make_cache(spec, "cpu", seed=0)
    cal = c.calib
    om = omega_np(64, spec.rope_theta)
    for h in range(spec.n_kv_heads):
        K = c.k[0][0, h].numpy().astype(np.float64)
        pos = c.pos[0][0, h].numpy().astype(np.int64)
        args = (cal.qc_re[0, h], cal.qc_im[0, h], cal.q_mean_norm[0, h], cal.q_mrl[0, h])
        trig, _, _ = oracle_lib.score_head(K, pos, c.p_now[0], om, cal.offsets, *args)
        q = qvec(cal.qc_re[0, h], cal.qc_im[0, h])
        brute = np.mean([K @ (rope_matrix(64, c.p_now[0] + int(dl), om) @ q)
                         for dl in cal.offsets], axis=0)
        np.testing.assert_allclose(trig, brute, atol=1e-10 * np.abs(brute).max())


def test_single_offset_is_the_rope_attention_logit(oracle_lib):
    """D = {delta}: the trig term is exactly q(p_now+delta) . k(p_i), the
    logit of RoPE attention, computed from pre-RoPE vectors."""
    rng = np.random.default_rng(5)
    d, n = 32, 20
    om = omega_np(d, 1e4)
    q = rng.standard_normal(d)
    k_pre = rng.standard_normal((n, d))
    pos = np.arange(100, 100 + 3 * n, 3, dtype=np.int64)
    K = np.stack([rope_matrix(d, int(p), om) @ k_pre[i] for i, p in enumerate(pos)])
    p_now, delta = 400, 9
    trig, _, _ = oracle_lib.score_head(K, pos, p_now, om, [delta], q[:16], q[16:],
                                       np.ones(16), np.ones(16))
    logit = np.array([(rope_matrix(d, p_now + delta, om) @ q) @ (rope_matrix(d, int(p), om) @ k_pre[i])
                      for i, p in enumerate(pos)])
    np.testing.assert_allclose(trig, logit, atol=1e-11)


def test_key_equal_to_centre_at_zero_distance_gives_squared_norm(oracle_lib):
    d = 16
    om = omega_np(d, 1e4)
    rng = np.random.default_rng(2)
    q = rng.standard_normal(d)
    p_now, delta = 1000, 64
    p = p_now + delta
    K = rope_matrix(d, p, om) @ q
    trig, norm, score = oracle_lib.score_head(K[None], [p], p_now, om, [delta], q[:8], q[8:],
                                              np.ones(8), np.ones(8))
    np.testing.assert_allclose(trig[0], q @ q, rtol=1e-12)
    assert norm[0] == 0.0


def test_zero_query_centre_gives_zero_trig(oracle_lib):
    rng = np.random.default_rng(3)
    d, n = 64, 30
    _, _, m, R, pos, K = random_head(rng, d, n)
    z = np.zeros(d // 2)
    trig, norm, score = oracle_lib.score_head(K, pos, 6000, omega_np(d, 1e4), [1, 2, 4], z, z, m, R)
    assert np.all(trig == 0.0)
    np.testing.assert_array_equal(score, norm)


def test_polar_per_band_form(oracle_lib):
    """Single band: trig = |q||k| * mean cos(w*dist + arg q - arg k), the
    pages' per-band form with phi the query/key phase difference."""
    rng = np.random.default_rng(4)
    om = np.array([0.37])
    for _ in range(20):
        rq, a = rng.uniform(0.1, 3), rng.uniform(-math.pi, math.pi)
        rk, b = rng.uniform(0.1, 3), rng.uniform(-math.pi, math.pi)
        p = int(rng.integers(0, 5000))
        p_now = p + int(rng.integers(0, 100))
        offs = [1, 2, 4, 8, 16, 32]
        k = np.array([rk * math.cos(b), rk * math.sin(b)])
        K = rope_matrix(2, p, om) @ k
        trig, _, _ = oracle_lib.score_head(K[None], [p], p_now, om, offs,
                                           [rq * math.cos(a)], [rq * math.sin(a)], [1.0], [1.0])
        expect = rq * rk * np.mean([math.cos(0.37 * (p_now + dl - p) + a - b) for dl in offs])
        assert abs(trig[0] - expect) <= 1e-12 * rq * rk


def test_trig_swapping_query_and_key_roles_is_detected(oracle_lib):
    """conj on the query instead of the key flips the phase; the oracle must
    follow q * conj(k) (query rotated to the later position)."""
    om = np.array([1.0])
    K = np.array([1.0, 0.0])      # k = 1 at position 0
    trig, _, _ = oracle_lib.score_head(K[None], [0], 0, om, [1], [0.0], [1.0], [1.0], [1.0])
    # q = i, dist = 1: Re(i * 1 * e^{i}) = -sin(1); the swapped form would give +sin(1)
    assert abs(trig[0] + math.sin(1.0)) < 1e-15


# ------------------------------------------------------------- norm term

def test_norm_term_special_cases_and_direct_sum(oracle_lib):
    rng = np.random.default_rng(6)
    d, n = 64, 25
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, n)
    om = omega_np(d, 1e4)
    h = d // 2
    band = np.hypot(K[:, :h], K[:, h:])           # |K_f| = |k_f| after any rotation
    _, norm1, _ = oracle_lib.score_head(K, pos, 6000, om, [1], qc_re, qc_im, m, np.ones(h))
    assert np.all(norm1 == 0.0)
    _, norm0, _ = oracle_lib.score_head(K, pos, 6000, om, [1], qc_re, qc_im, m, np.zeros(h))
    np.testing.assert_allclose(norm0, band @ m, rtol=1e-13)
    _, norm, _ = oracle_lib.score_head(K, pos, 6000, om, [1], qc_re, qc_im, m, R)
    np.testing.assert_allclose(norm, band @ ((1 - R) * m), rtol=1e-13)


def test_norm_term_is_position_invariant(oracle_lib):
    rng = np.random.default_rng(7)
    d = 32
    om = omega_np(d, 1e4)
    k = rng.standard_normal(d)
    qr, qi = rng.standard_normal(16), rng.standard_normal(16)
    m, R = rng.uniform(1, 2, 16), rng.uniform(0, 1, 16)
    norms = []
    for p in [0, 17, 999, 123456]:
        _, nm, _ = oracle_lib.score_head((rope_matrix(d, p, om) @ k)[None], [p], 200000, om,
                                         [1, 2], qr, qi, m, R)
        norms.append(nm[0])
    np.testing.assert_allclose(norms, norms[0], rtol=1e-13)


def test_score_is_sum_and_bounded(oracle_lib):
    rng = np.random.default_rng(8)
    d, n = 128, 50
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, n)
    om = omega_np(d, 5e5)
    offs = synth.pow2_offsets(16)
    trig, norm, score = oracle_lib.score_head(K, pos, 5000, om, offs, qc_re, qc_im, m, R)
    np.testing.assert_array_equal(score, trig + norm)
    M = oracle_lib.bound_head(K, om, offs, qc_re, qc_im, m, R)
    assert np.all(np.abs(score) <= M * (1 + 1e-12))


def test_folded_form_agrees(oracle_lib):
    """Independent second derivation: with A_f = mean_delta e^{i w_f delta} and
    C_f = qc_f * A_f * e^{i w_f p_now}, the score is the plain dot product
    [Re C; Im C] . K plus sum_f w_f |K_f| on the stored row (no inverse RoPE)."""
    rng = np.random.default_rng(9)
    d, n = 128, 64
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, n, pmax=32768)
    om = omega_np(d, 1e6)
    offs = np.array(synth.pow2_offsets(16))
    p_now = 32767
    A = np.exp(1j * np.outer(om, offs)).mean(axis=1)
    C = (qc_re + 1j * qc_im) * A * np.exp(1j * om * p_now)
    u = np.concatenate([C.real, C.imag])
    h = d // 2
    folded = K @ u + np.hypot(K[:, :h], K[:, h:]) @ ((1 - R) * m)
    _, _, score = oracle_lib.score_head(K, pos, p_now, om, offs, qc_re, qc_im, m, R)
    M = oracle_lib.bound_head(K, om, offs, qc_re, qc_im, m, R)
    assert np.all(np.abs(score - folded) <= 1e-11 * M)


# ------------------------------------------- the tolerance scale M, two-sided

def _bound_golden():
    with open(os.path.join(GOLDEN, "bound_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("i", range(len(_bound_golden()["examples"])))
def test_golden_bound_examples(oracle_lib, i):
    """Hand-derived values of M (tests/golden/bound_examples.json)."""
    ex = _bound_golden()["examples"][i]
    d = ex["head_dim"]
    qc = np.array(ex["qc"])
    M = oracle_lib.bound_head(np.array([ex["key_stored"]]), ex["omega"], ex["offsets"],
                              qc[: d // 2], qc[d // 2:], ex["q_mean_norm"], ex["q_mrl"])
    assert abs(M[0] - ex["bound"]) <= 1e-12 * max(1.0, abs(ex["bound"]))


@pytest.mark.parametrize("seed", range(6))
def test_bound_is_the_largest_score_over_key_phases(oracle_lib, seed):
    """M is attained: with one band, the score of a key of fixed magnitude r
    is a + b cos(phi) + c sin(phi) in the stored phase phi (the trig term is
    linear in the stored row, the norm term does not see the phase), so its
    largest value over phi is a + sqrt(b^2 + c^2).  Four phases give a, b, c
    from the oracle's own scores, a fifth checks the form; M must equal that
    maximum, and the smallest score must be 2a - M."""
    rng = np.random.default_rng(100 + seed)
    om = rng.uniform(0.01, 3.0, 1)
    offs = np.sort(rng.choice(1 << 12, size=int(rng.integers(1, 6)), replace=False)) + 1
    qr, qi = rng.standard_normal(1), rng.standard_normal(1)
    m = np.hypot(qr, qi) * rng.uniform(1.0, 2.0, 1)
    R = rng.uniform(0.0, 1.0, 1)
    r = rng.uniform(0.5, 3.0)
    p, p_now = int(rng.integers(0, 4000)), 4000 + int(rng.integers(0, 100))

    def s_at(phi):
        K = np.array([[r * math.cos(phi), r * math.sin(phi)]])
        return oracle_lib.score_head(K, [p], p_now, om, offs, qr, qi, m, R)[2][0]

    s0, s1, s2, s3 = (s_at(k * math.pi / 2) for k in range(4))
    a, b, c = (s0 + s1 + s2 + s3) / 4, (s0 - s2) / 2, (s1 - s3) / 2
    phi = 0.7
    assert abs(s_at(phi) - (a + b * math.cos(phi) + c * math.sin(phi))) <= 1e-12 * (abs(a) + abs(b) + abs(c))
    top = a + math.hypot(b, c)
    M = oracle_lib.bound_head(np.array([[r, 0.0]]), om, offs, qr, qi, m, R)[0]
    assert abs(M - top) <= 1e-12 * M
    assert abs((2 * a - M) - (a - math.hypot(b, c))) <= 1e-12 * M
    assert abs(a - (1 - R[0]) * m[0] * r) <= 1e-12 * M      # the phase-free part is the norm term


def test_bound_adds_over_bands(oracle_lib):
    """M of a key is the sum of M over its bands taken one at a time (every
    other band zero), and it scales with the key: M(cK) = |c| M(K)."""
    rng = np.random.default_rng(11)
    d = 8
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, 5)
    om = omega_np(d, 1e4)
    offs = synth.pow2_offsets(10)
    M = oracle_lib.bound_head(K, om, offs, qc_re, qc_im, m, R)
    h = d // 2
    parts = np.zeros(len(K))
    for f in range(h):
        Kf = np.zeros_like(K)
        Kf[:, f], Kf[:, f + h] = K[:, f], K[:, f + h]
        parts += oracle_lib.bound_head(Kf, om, offs, qc_re, qc_im, m, R)
    np.testing.assert_allclose(M, parts, rtol=1e-13)
    np.testing.assert_allclose(oracle_lib.bound_head(-2.5 * K, om, offs, qc_re, qc_im, m, R), 2.5 * M,
                               rtol=1e-13)


# ------------------------------------------------------- non-finite keys

def test_nonfinite_keys_score_nan_and_are_evicted(oracle_lib):
    """A key whose stored row holds +inf, -inf or NaN scores NaN (trig, norm
    and score), so it ranks below every number; the other keys score as they
    would alone.  The one-band case K = (inf, inf), centre 1, R = 0 is one
    where plain complex arithmetic reaches +inf, which would rank first."""
    t, nm, s = oracle_lib.score_head(np.array([[np.inf, np.inf]]), [0], 0, [1.0], [1],
                                     [1.0], [0.0], [1.0], [0.0])
    assert np.isnan(t[0]) and np.isnan(nm[0]) and np.isnan(s[0])
    rng = np.random.default_rng(12)
    d, n = 128, 40
    qc_re, qc_im, m, R, pos, K = random_head(rng, d, n)
    om = omega_np(d, 1e6)
    offs = synth.pow2_offsets(16)
    bad = {3: np.inf, 7: -np.inf, 11: np.nan, 20: np.inf, 33: np.nan}
    Kb = K.copy()
    for i, v in bad.items():
        Kb[i, int(rng.integers(0, d))] = v
    Kb[20, 5], Kb[20, 5 + d // 2] = np.inf, -np.inf
    trig, norm, score = oracle_lib.score_head(Kb, pos, 6000, om, offs, qc_re, qc_im, m, R)
    good = np.array([i not in bad for i in range(n)])
    for x in (trig, norm, score):
        assert np.all(np.isnan(x[~good])) and np.all(np.isfinite(x[good]))
    _, _, alone = oracle_lib.score_head(K[good], pos[good], 6000, om, offs, qc_re, qc_im, m, R)
    np.testing.assert_array_equal(score[good], alone)
    kept = oracle_lib.select_head(score, pos, n - len(bad), 0)
    assert sorted(kept.tolist()) == np.nonzero(good)[0].tolist()


# --------------------------------------------------------- golden examples

def _golden():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def _num(x):
    return float(x) if not isinstance(x, str) else float(x)


@pytest.mark.parametrize("ex", _golden()["score_examples"], ids=lambda e: e["name"])
def test_golden_score_examples(oracle_lib, ex):
    d = ex["head_dim"]
    om = np.array(ex["omega"])
    k = np.array(ex["key_pre_rope"])
    K = rope_matrix(d, ex["pos"], om) @ k
    qc = np.array(ex["qc"])
    trig, norm, score = oracle_lib.score_head(K[None], [ex["pos"]], ex["p_now"], om, ex["offsets"],
                                              qc[: d // 2], qc[d // 2:], ex["q_mean_norm"], ex["q_mrl"])
    assert abs(trig[0] - ex["trig"]) < 1e-13
    assert abs(norm[0] - ex["norm"]) < 1e-13
    assert abs(score[0] - ex["score"]) < 1e-13


@pytest.mark.parametrize("i", range(len(_golden()["select_examples"])))
def test_golden_select_examples(oracle_lib, i):
    ex = _golden()["select_examples"][i]
    s = np.array([_num(x) for x in ex["scores"]])
    kept = oracle_lib.select_head(s, ex["pos"], ex["budget"], ex["window"])
    if ex["kept"] is None:
        assert kept is None
    else:
        assert kept.tolist() == ex["kept"]


def test_pages_constants_match_workloads():
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        pc = json.load(f)
    assert list(synth.pow2_offsets(16)) == pc["offsets"]
    assert len(pc["offsets"]) == 17
    for name in ("llama8b", "qwen3_32k", "batched", "wide"):
        spec = synth.workload(name)
        assert list(spec.offsets) == pc["offsets"]
        assert spec.window == pc["window"]
    assert synth.workload("llama8b").budget == pc["default_budget"]
    assert abs(pc["max_generation_tokens"] / pc["aime25_matched_budget"] - pc["kv_reduction"]) < 0.05


# ---------------------------------------------------------------- top-B

def _beats(si, pi, sj, pj):
    """True when key i ranks above key j: larger score, NaN lowest, ties by position."""
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni != nj:
        return nj
    if not ni and si != sj:
        return si > sj
    return pi < pj


@pytest.mark.parametrize("seed", range(12))
def test_select_equals_bruteforce_subset_search(oracle_lib, seed):
    """The kept set is the unique subset whose every member beats every
    evicted key; found by enumerating all subsets of a tiny head."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 10))
    B = int(rng.integers(1, n))
    vals = np.array([-1.0, 0.0, -0.0, 0.5, 2.0, np.nan, np.inf])
    s = rng.choice(vals, size=n) if seed % 2 else rng.standard_normal(n).round(1)
    pos = rng.permutation(100)[:n].astype(np.int64)
    winners = [S for S in itertools.combinations(range(n), B)
               if all(_beats(s[i], pos[i], s[j], pos[j])
                      for i in S for j in range(n) if j not in S)]
    assert len(winners) == 1
    kept = oracle_lib.select_head(s, pos, B, 0)
    assert kept.tolist() == list(winners[0])


def test_select_matches_numpy_lexsort(oracle_lib):
    rng = np.random.default_rng(11)
    n, B = 5000, 700
    s = rng.choice(np.linspace(-3, 3, 41), size=n)       # many ties
    pos = np.sort(rng.choice(100000, size=n, replace=False)).astype(np.int64)
    order = np.lexsort((pos, -s))                          # score desc, then position asc
    expect = np.sort(order[:B])
    np.testing.assert_array_equal(oracle_lib.select_head(s, pos, B, 128), expect)


def test_select_invariants_and_fire_rule(oracle_lib):
    rng = np.random.default_rng(12)
    n = 1000
    s = rng.standard_normal(n)
    pos = np.arange(n, dtype=np.int64)
    assert oracle_lib.select_head(s, pos, 900, 100) is None          # 1000 = 900 + 100
    kept = oracle_lib.select_head(s, pos, 899, 100)
    assert len(kept) == 899 and np.all(np.diff(kept) > 0)
    ev = np.setdiff1d(np.arange(n), kept)
    assert s[kept].min() >= s[ev].max()
    allsame = oracle_lib.select_head(np.full(n, 2.5), pos, 10, 0)
    np.testing.assert_array_equal(allsame, np.arange(10))


# ------------------------------------------------------------- gather

def test_gather_matches_numpy_take_and_identity(oracle_lib):
    rng = np.random.default_rng(13)
    rows = rng.standard_normal((300, 64)).astype(np.float32)
    kept = np.sort(rng.choice(300, 77, replace=False)).astype(np.int32)
    np.testing.assert_array_equal(oracle_lib.gather_rows(kept, rows), rows[kept])
    np.testing.assert_array_equal(oracle_lib.gather_rows(np.arange(50), rows), rows[:50])
    p = np.arange(300, dtype=np.int32) * 3
    np.testing.assert_array_equal(oracle_lib.gather_rows(kept, p), p[kept])


def test_prune_head_end_to_end_small(oracle_lib):
    """Score, select and gather on one toy head: the kept rows are the
    top-B by score (ties by position), copied bit-exactly in slot order."""
    spec = synth.workload("toy")
    c = synth.make_cache(spec, "cpu", seed=3)
    cal = c.calib
    om = oracle_lib.omega(64, spec.rope_theta)
    K = c.k[0][0, 1].numpy()
    V = c.v[0][0, 1].numpy()
    pos = c.pos[0][0, 1].numpy()
    r = oracle_lib.prune_head(K, V, pos, c.p_now[0], om, cal.offsets, cal.qc_re[0, 1],
                              cal.qc_im[0, 1], cal.q_mean_norm[0, 1], cal.q_mrl[0, 1],
                              spec.budget, spec.window)
    order = np.lexsort((pos, -r["score"]))
    np.testing.assert_array_equal(r["kept"], np.sort(order[: spec.budget]))
    np.testing.assert_array_equal(r["K"], K[r["kept"]])
    np.testing.assert_array_equal(r["V"], V[r["kept"]])
    np.testing.assert_array_equal(r["pos"], pos[r["kept"]])
