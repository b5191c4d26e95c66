"""Pins of the oracle's GQA normalize-then-aggregate score.

Source: dimensionstp.github.io TriAttention review, section 3-2 item 6, and
romaanj.github.io TriAttention review, section "Method": query heads that
share a KV head each z-normalize their key scores, and a key's score is the
max over those query heads.  The pins are hand-derived closed forms
(tests/golden/gqa_examples.json), properties every z-score has (zero mean,
unit population variance, invariance to each query head's scale), the
single-query-head case reducing to the plain ranking, and the treatment of
degenerate rows.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "gqa_examples.json")) as f:
        return json.load(f)


def _num(x):
    return float("nan") if x == "nan" else float(x)


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(y) for y in x], dtype=np.float64)
    return _num(x)


def _close_nan(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    assert np.array_equal(np.isnan(a), np.isnan(b))
    m = ~np.isnan(a)
    np.testing.assert_allclose(a[m], b[m], rtol=0, atol=tol)


def _random_group(rng, d, n, G, pmax=4000):
    h = d // 2
    qc_re = rng.standard_normal((G, h))
    qc_im = rng.standard_normal((G, h))
    m = np.hypot(qc_re, qc_im) * (1 + rng.uniform(0, 0.5, (G, h)))
    R = np.hypot(qc_re, qc_im) / m
    pos = np.sort(rng.choice(pmax, size=n, replace=False)).astype(np.int64)
    K = rng.standard_normal((n, d))
    return qc_re, qc_im, m, R, pos, K


@pytest.mark.parametrize("i", range(3))
def test_gqa_golden_examples(oracle_lib, i):
    ex = _golden()["examples"][i]
    K = _arr(ex["keys"])
    pos = np.array(ex["pos"], dtype=np.int64)
    qc = _arr(ex["qc"])
    raw, z, score = oracle_lib.gqa_head(K, pos, ex["p_now"], np.array(ex["omega"]), ex["offsets"],
                                        qc[:, :1], qc[:, 1:], _arr(ex["q_mean_norm"]),
                                        _arr(ex["q_mrl"]))
    _close_nan(raw, _arr(ex["raw"]), 1e-13)
    _close_nan(z, _arr(ex["z"]), 1e-13)
    _close_nan(score, _arr(ex["score"]), 1e-13)
    kept = oracle_lib.select_head(score, pos, ex["budget"], ex["window"])
    assert list(kept) == ex["kept"]


def test_gqa_z_rows_have_zero_mean_and_unit_population_variance(oracle_lib):
    rng = np.random.default_rng(7)
    qr, qi, m, R, pos, K = _random_group(rng, 16, 300, 4)
    om = oracle_lib.omega(16, 1e4)
    raw, z, score = oracle_lib.gqa_head(K, pos, 4000, om, [1, 2, 4, 8], qr, qi, m, R)
    for g in range(4):
        assert abs(z[g].mean()) < 1e-12
        assert abs((z[g] ** 2).mean() - 1.0) < 1e-12
        # z is an increasing affine map of the raw row
        order = np.argsort(raw[g], kind="stable")
        assert np.all(np.diff(z[g][order]) >= -1e-12)
    np.testing.assert_array_equal(score, z.max(axis=0))


def test_gqa_score_is_free_of_each_query_heads_scale(oracle_lib):
    rng = np.random.default_rng(8)
    qr, qi, m, R, pos, K = _random_group(rng, 16, 200, 1)
    c = 3.7
    qr2 = np.vstack([qr, c * qr])
    qi2 = np.vstack([qi, c * qi])
    m2 = np.vstack([m, c * m])
    R2 = np.vstack([R, R])
    om = oracle_lib.omega(16, 1e4)
    raw, z, score = oracle_lib.gqa_head(K, pos, 4000, om, [1, 2, 4], qr2, qi2, m2, R2)
    np.testing.assert_allclose(raw[1], c * raw[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z[1], z[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(score, z[0], rtol=0, atol=1e-12)


def test_gqa_single_query_head_keeps_the_plain_top_b(oracle_lib):
    rng = np.random.default_rng(9)
    qr, qi, m, R, pos, K = _random_group(rng, 32, 400, 1)
    om = oracle_lib.omega(32, 1e4)
    _, _, plain = oracle_lib.score_head(K, pos, 4000, om, [1, 2, 4, 8, 16], qr[0], qi[0], m[0], R[0])
    raw, z, score = oracle_lib.gqa_head(K, pos, 4000, om, [1, 2, 4, 8, 16], qr, qi, m, R)
    np.testing.assert_array_equal(raw[0], plain)
    a = oracle_lib.select_head(plain, pos, 100, 10)
    b = oracle_lib.select_head(score, pos, 100, 10)
    np.testing.assert_array_equal(a, b)


def test_gqa_equal_scores_give_zero(oracle_lib):
    rng = np.random.default_rng(10)
    qr, qi, m, R, pos, K = _random_group(rng, 8, 50, 3)
    K[:] = K[0]
    pos[:] = 100              # same stored row at the same position: equal scores
    om = oracle_lib.omega(8, 1e4)
    raw, z, score = oracle_lib.gqa_head(K, pos, 200, om, [1, 2], qr, qi, m, R)
    assert np.all(raw == raw[:, :1])
    assert np.all(z == 0.0) and np.all(score == 0.0)


def test_gqa_nonfinite_key_is_left_out_of_the_statistics(oracle_lib):
    rng = np.random.default_rng(11)
    qr, qi, m, R, pos, K = _random_group(rng, 16, 120, 2)
    om = oracle_lib.omega(16, 1e4)
    bad = 37
    K_bad = K.copy()
    K_bad[bad, 3] = np.inf
    _, z_all, s_all = oracle_lib.gqa_head(K_bad, pos, 4000, om, [1, 4], qr, qi, m, R)
    keep = np.arange(120) != bad
    _, z_ref, s_ref = oracle_lib.gqa_head(K[keep], pos[keep], 4000, om, [1, 4], qr, qi, m, R)
    assert math.isnan(s_all[bad]) and np.all(np.isnan(z_all[:, bad]))
    np.testing.assert_allclose(z_all[:, keep], z_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s_all[keep], s_ref, rtol=0, atol=1e-12)


def test_gqa_max_over_the_group_of_separately_normalized_heads(oracle_lib):
    rng = np.random.default_rng(12)
    qr, qi, m, R, pos, K = _random_group(rng, 16, 150, 3)
    om = oracle_lib.omega(16, 1e4)
    _, _, score = oracle_lib.gqa_head(K, pos, 4000, om, [1, 2, 4], qr, qi, m, R)
    each = [oracle_lib.gqa_head(K, pos, 4000, om, [1, 2, 4], qr[g:g + 1], qi[g:g + 1],
                                m[g:g + 1], R[g:g + 1])[2] for g in range(3)]
    np.testing.assert_array_equal(score, np.max(np.vstack(each), axis=0))


def test_gqa_z_rows_equal_a_library_zscore(oracle_lib):
    """The per-query-head normalization against a library routine
    (scipy.stats.zscore, population deviation) over the finite scores of each
    row; a key with a non-finite element has NaN in every row."""
    stats = pytest.importorskip("scipy.stats")
    rng = np.random.default_rng(11)
    qr, qi, m, R, pos, K = _random_group(rng, 16, 257, 4)
    K[[5, 100]] = np.nan
    K[200, 3] = np.inf
    om = oracle_lib.omega(16, 1e4)
    raw, z, score = oracle_lib.gqa_head(K, pos, 5000, om, [1, 2, 4, 8, 16], qr, qi, m, R)
    fin = np.isfinite(K).all(axis=1)
    for g in range(4):
        assert np.all(np.isnan(z[g][~fin]))
        np.testing.assert_allclose(z[g][fin], stats.zscore(raw[g][fin], ddof=0), rtol=0, atol=1e-12)
    assert np.all(np.isnan(score[~fin]))
    np.testing.assert_array_equal(score[fin], np.max(z[:, fin], axis=0))
