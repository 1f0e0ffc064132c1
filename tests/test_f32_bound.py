"""The fp32 tolerance of the random-shape sweep (helpers.assert_f32_within)
admits an fp32 evaluation of the layer and rejects one with a term or a
token row left out (CPU; numpy's fp32 products stand in for a correct fp32
implementation, the oracle gives the exact values and the magnitudes)."""
import numpy as np
import pytest

from tests.helpers import assert_f32_within, gamma_prob_f32


def test_gamma_prob_small_n():
    # lam sqrt(n) u dominates: g~_n ~= 8 sqrt(n) 2^-24
    assert gamma_prob_f32(1) == pytest.approx(8 * 2.0 ** -24, rel=1e-6)
    assert gamma_prob_f32(10000) == pytest.approx(800 * 2.0 ** -24, rel=1e-4)


def _case(orc, M, N, K, r, alpha, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    A = (0.01 * rng.standard_normal((r, K))).astype(np.float32)
    B = (0.01 * rng.standard_normal((N, r))).astype(np.float32)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    _, dA_ref, dB_ref = orc.linear_bwd(x, w, A, B, dy, alpha, r, want_dx=False)
    ab = np.abs
    _, dA_mag, _ = orc.linear_bwd(ab(x), ab(w), ab(A), ab(B), ab(dy), alpha, r, want_dx=False)
    s = np.float32(alpha) / np.float32(r)
    g = s * (dy @ B)
    return x, g, dA_ref, dA_mag


def test_f32_bound_admits_fp32_and_rejects_a_dropped_row(orc):
    M, N, K, r = 300, 1536, 512, 32
    x, g, dA_ref, dA_mag = _case(orc, M, N, K, r, 64.0, 5)
    n = N + 1 + M + 4
    assert_f32_within(g.T @ x, dA_ref, dA_mag, n, "dA")
    with pytest.raises(AssertionError):
        assert_f32_within(g[:-1].T @ x[:-1], dA_ref, dA_mag, n, "dA without the last row")
    bad = (g.T @ x).copy()
    terms = g[:, 3].astype(np.float64) * x[:, 7]
    m = int(np.argsort(np.abs(terms))[M // 2])          # the median-size term
    bad[3, 7] += np.float32(terms[m])
    with pytest.raises(AssertionError):
        assert_f32_within(bad, dA_ref, dA_mag, n, "dA with one term doubled")
