"""Pins of the oracle's calibration statistics from pre-RoPE query samples.

Source: romaanj.github.io TriAttention review, section "Method" (per band:
the pre-RoPE query centre E[q_f], the mean norm and the mean resultant
length R_f from a calibration pass); dimensionstp.github.io TriAttention
review, section 3 (calibration phase; concentration measured as MRL).
Reading: R_f = |E[q_f]| / E|q_f|.  The pins are hand-derived examples
(tests/golden/calib_examples.json), closed forms (equal samples give R = 1,
opposite samples R = 0), the wrapped-normal law E[e^{i theta}] =
e^{i mu - sigma^2 / 2} checked statistically on samples of known
concentration, and invariance to scaling and to a common rotation.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "calib_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("i", range(4))
def test_calib_golden_examples(oracle_lib, i):
    ex = _golden()["examples"][i]
    qr, qi, m, R = oracle_lib.calib_stats(np.array(ex["samples"]))
    for got, key in ((qr, "qc_re"), (qi, "qc_im"), (m, "q_mean_norm"), (R, "q_mrl")):
        np.testing.assert_allclose(got, ex[key], rtol=0, atol=1e-14)


def test_calib_equal_and_opposite_samples(oracle_lib):
    rng = np.random.default_rng(20)
    row = rng.standard_normal(16)
    qr, qi, m, R = oracle_lib.calib_stats(np.tile(row, (9, 1)))
    np.testing.assert_allclose(qr, row[:8], atol=1e-14)
    np.testing.assert_allclose(qi, row[8:], atol=1e-14)
    np.testing.assert_allclose(m, np.hypot(row[:8], row[8:]), atol=1e-14)
    np.testing.assert_allclose(R, 1.0, atol=1e-14)
    qr, qi, m, R = oracle_lib.calib_stats(np.vstack([row, -row]))
    assert np.all(np.abs(qr) < 1e-15) and np.all(np.abs(qi) < 1e-15)
    assert np.all(R < 1e-14)


def test_calib_recovers_a_known_concentration(oracle_lib):
    """Phases mu + N(0, sigma^2) at constant magnitude: E[e^{i theta}] = e^{i mu - sigma^2/2},
    so R = exp(-sigma^2 / 2) and arg E[q] = mu; n = 200000 samples, error ~ 1/sqrt(n)."""
    rng = np.random.default_rng(21)
    h, n = 6, 200_000
    mu = rng.uniform(-np.pi, np.pi, h)
    R_true = np.array([0.99, 0.95, 0.8, 0.6, 0.3, 0.1])
    sigma = np.sqrt(-2.0 * np.log(R_true))
    mag = rng.uniform(0.5, 3.0, h)
    theta = mu + sigma * rng.standard_normal((n, h))
    Q = np.hstack([mag * np.cos(theta), mag * np.sin(theta)])
    qr, qi, m, R = oracle_lib.calib_stats(Q)
    np.testing.assert_allclose(R, R_true, atol=0.01)
    np.testing.assert_allclose(m, mag, rtol=1e-10)
    ang = np.angle((qr + 1j * qi) * np.exp(-1j * mu))
    assert np.all(np.abs(ang[R_true > 0.5]) < 0.01)


def test_calib_scale_and_rotation(oracle_lib):
    rng = np.random.default_rng(22)
    Q = rng.standard_normal((500, 8)) + np.array([2.0, -1.0, 0.5, 0.0, 1.0, 1.0, -2.0, 0.3])
    qr, qi, m, R = oracle_lib.calib_stats(Q)
    qr2, qi2, m2, R2 = oracle_lib.calib_stats(2.5 * Q)
    np.testing.assert_allclose(qr2, 2.5 * qr, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(m2, 2.5 * m, rtol=1e-13)
    np.testing.assert_allclose(R2, R, rtol=1e-13)
    phi = np.array([0.3, -1.2, 2.0, 0.7])
    c, s = np.cos(phi), np.sin(phi)
    a, b = Q[:, :4], Q[:, 4:]
    Qr = np.hstack([a * c - b * s, a * s + b * c])
    qr3, qi3, m3, R3 = oracle_lib.calib_stats(Qr)
    np.testing.assert_allclose(qr3 + 1j * qi3, (qr + 1j * qi) * np.exp(1j * phi), atol=1e-13)
    np.testing.assert_allclose(m3, m, rtol=1e-13)
    np.testing.assert_allclose(R3, R, rtol=1e-12)
