"""Pins of the oracle's distance-preference curve and future-offset sets.

Sources: dimensionstp.github.io TriAttention review, section 2-1 item 2 (Q/K
centres give a distance preference curve), section 2-2 (the RoPE logit
a(i, j) = sum_f r_q r_k cos((i - j) theta_f + phi_f)), section 4-3 "Future
offset design" (maximum distance and spacing; geometric beats linear),
section 6 item 2 (per-head curves as an analysis tool); romaanj.github.io
TriAttention review, section "Method" (offsets {1, 2, 4, ..., 2^16}).
The curve is pinned to dense RoPE rotation matrices (the logit of a query
at the centre and a key at the centre delta positions earlier), to its
value at delta 0, to a hand example, and to the score's trigonometric term
of a key that sits exactly at the centre.  CPU only.
"""
import math

import numpy as np

from test_oracle_pins import omega_np, rope_matrix


def _pair(rng, d):
    h = d // 2
    return rng.standard_normal(h), rng.standard_normal(h), rng.standard_normal(h), rng.standard_normal(h)


def test_curve_is_the_rope_logit_of_the_centres(oracle_lib):
    rng = np.random.default_rng(30)
    for d, theta in ((8, 10.0), (64, 1e4), (128, 1e6)):
        qr, qi, kr, ki = _pair(rng, d)
        om = omega_np(d, theta)
        deltas = np.array([0, 1, 2, 7, 100, 4096, 65536, -5], dtype=np.int64)
        got = oracle_lib.distance_curve(om, qr, qi, kr, ki, deltas)
        q = np.concatenate([qr, qi])
        k = np.concatenate([kr, ki])
        i = 70001
        for dj, g in zip(deltas, got):
            ref = (rope_matrix(d, i, om) @ q) @ (rope_matrix(d, i - int(dj), om) @ k)
            assert abs(g - ref) <= 1e-9 * (1 + abs(ref))


def test_curve_at_zero_distance_is_the_dot_product_and_hand_example(oracle_lib):
    rng = np.random.default_rng(31)
    qr, qi, kr, ki = _pair(rng, 16)
    om = omega_np(16, 1e4)
    s0 = oracle_lib.distance_curve(om, qr, qi, kr, ki, [0])[0]
    assert abs(s0 - (qr @ kr + qi @ ki)) < 1e-12
    # one band, w = 0.5, q = 2, k = 1 + i: Re(2 (1 - i) e^{i x}) = 2 (cos x + sin x), x = delta / 2
    got = oracle_lib.distance_curve([0.5], [2.0], [0.0], [1.0], [1.0], [0, 1, 4])
    ref = [2 * (math.cos(x) + math.sin(x)) for x in (0.0, 0.5, 2.0)]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_score_trig_term_of_a_key_at_the_centre_averages_the_curve(oracle_lib):
    rng = np.random.default_rng(32)
    d, theta = 32, 5e5
    qr, qi, kr, ki = _pair(rng, d)
    om = omega_np(d, theta)
    pos = np.array([10, 500, 3000, 40000], dtype=np.int64)
    K = np.stack([rope_matrix(d, int(p), om) @ np.concatenate([kr, ki]) for p in pos])
    offsets = np.array([1, 2, 4, 8, 16, 1024], dtype=np.int64)
    p_now = 50000
    m = np.ones(d // 2)
    R = np.ones(d // 2)            # no norm term
    trig, _, _ = oracle_lib.score_head(K, pos, p_now, om, offsets, qr, qi, m, R)
    for i, p in enumerate(pos):
        c = oracle_lib.distance_curve(om, qr, qi, kr, ki, p_now + offsets - p)
        assert abs(trig[i] - c.mean()) <= 1e-9 * (1 + abs(c.mean()))


def test_offset_sets(oracle_lib):
    geo = oracle_lib.offset_set("geometric", 65536)
    np.testing.assert_array_equal(geo, [2 ** e for e in range(17)])   # the pages' {1, 2, ..., 2^16}
    np.testing.assert_array_equal(oracle_lib.offset_set("geometric", 100), [1, 2, 4, 8, 16, 32, 64])
    # 1000 * k / 7 rounded: 142.9, 285.7, 428.6, 571.4, 714.3, 857.1, 1000
    np.testing.assert_array_equal(oracle_lib.offset_set("linear", 1000, 7),
                                  [143, 286, 429, 571, 714, 857, 1000])
    np.testing.assert_array_equal(oracle_lib.offset_set("linear", 3, 6), [1, 1, 2, 2, 3, 3])


def test_curve_is_the_logit_of_a_model_librarys_rope(oracle_lib):
    """The curve with the oracle's own frequencies against a model library's
    RoPE (the Llama rotary embedding of `transformers`): the dot product of
    the query centre rotated to position i + delta and the key centre rotated
    to position i (the library computes its angles in fp32, so positions stay
    small)."""
    from test_oracle_pins import _library_rope
    rng = np.random.default_rng(31)
    for d, theta in ((64, 1e4), (128, 1e6)):
        _, rotate = _library_rope(d, theta)
        qr, qi, kr, ki = _pair(rng, d)
        q = np.concatenate([qr, qi])
        k = np.concatenate([kr, ki])
        deltas = np.array([0, 1, 2, 7, 40, 100, -5], dtype=np.int64)
        got = oracle_lib.distance_curve(oracle_lib.omega(d, theta), qr, qi, kr, ki, deltas)
        i = 120
        kk = rotate(k[None], [i])[0]
        for dj, g in zip(deltas, got):
            ref = float(rotate(q[None], [i + int(dj)])[0] @ kk)
            assert abs(g - ref) <= 1e-6 * np.abs(q).sum() * np.abs(k).sum(), (d, dj, g, ref)
