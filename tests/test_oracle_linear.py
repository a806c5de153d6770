"""Pins of the oracle's reward scan, error estimate and outer product (no GPU).

Paper digest, section 2.2: r_t = sum_{s>=t} gamma^(s-t) c_s (gamma = 0: the
token's own c); g_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i); G_W = sum_t g_t x_t^T.
Pinned against:
  - gamma = 0: r == c bitwise; gamma = 1: a reversed cumulative sum per
    sequence (numpy); general gamma: the direct O(L^2) sum; a change inside one
    sequence leaves every other sequence untouched;
  - a one-hot c gives the closed form g_t = -(1/(K sigma)) gamma^(s*-t) a^(i*)_t
    for t <= s* in s*'s sequence and 0 elsewhere, with the noise from the
    (separately pinned) noise stream;
  - linearity in c and the 1/sigma scaling;
  - G_W against numpy's matmul, and a rank-one G_W for a single token.
"""
import numpy as np
import pytest

import oracle


def _direct_scan(c, L, gamma):
    K, T = c.shape
    r = np.zeros_like(c)
    for t in range(T):
        end = (t // L + 1) * L
        for s in range(t, end):
            r[:, t] += gamma ** (s - t) * c[:, s]
    return r


@pytest.mark.parametrize("L", [1, 5, 12])
def test_scan_special_cases(L):
    rng = np.random.default_rng(L)
    c = rng.standard_normal((3, 60))
    assert np.array_equal(oracle.reward_scan(c, L, 0.0), c)
    ref = np.concatenate([np.cumsum(c[:, s:s + L][:, ::-1], axis=1)[:, ::-1]
                          for s in range(0, 60, L)], axis=1)
    np.testing.assert_allclose(oracle.reward_scan(c, L, 1.0), ref, rtol=1e-12, atol=1e-12)
    for g in (0.3, 0.9):
        np.testing.assert_allclose(oracle.reward_scan(c, L, g), _direct_scan(c, L, g),
                                   rtol=1e-12, atol=1e-12)


def test_scan_segment_isolation():
    rng = np.random.default_rng(0)
    c = rng.standard_normal((2, 30))
    r0 = oracle.reward_scan(c, 10, 0.8)
    c2 = c.copy()
    c2[1, 14] += 5.0
    r1 = oracle.reward_scan(c2, 10, 0.8)
    diff = r1 != r0
    assert not diff[0].any()
    assert set(np.nonzero(diff[1])[0]) == set(range(10, 15))


@pytest.mark.parametrize("gamma", [0.0, 0.6])
def test_one_hot_reward_closed_form(gamma):
    K, T, L, N, d, sigma, seed, stream = 4, 12, 6, 8, 3, 0.25, 3, 1
    X = np.random.default_rng(1).standard_normal((T, d))
    a = oracle.noise(seed, stream, 0, K, T, N)
    for (i_s, s_s) in ((2, 9), (0, 0), (3, 5)):
        c = np.zeros((K, T))
        c[i_s, s_s] = 1.0
        g, G = oracle.linear_estimate(X, c, L, N, sigma, gamma, seed, stream)
        ref = np.zeros((T, N))
        seg0 = (s_s // L) * L
        for t in range(seg0, s_s + 1):
            ref[t] = -(gamma ** (s_s - t)) * a[i_s, t] / (K * sigma)
        np.testing.assert_allclose(g, ref, rtol=1e-12, atol=1e-15)


def test_linearity_and_sigma_scaling():
    K, T, L, N, d = 5, 8, 4, 12, 3
    rng = np.random.default_rng(2)
    X = rng.standard_normal((T, d))
    c1 = rng.standard_normal((K, T))
    c2 = rng.standard_normal((K, T))
    g1, G1 = oracle.linear_estimate(X, c1, L, N, 0.1, 0.5, 4)
    g2, G2 = oracle.linear_estimate(X, c2, L, N, 0.1, 0.5, 4)
    g3, G3 = oracle.linear_estimate(X, 2.0 * c1 - 3.0 * c2, L, N, 0.1, 0.5, 4)
    np.testing.assert_allclose(g3, 2 * g1 - 3 * g2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(G3, 2 * G1 - 3 * G2, rtol=1e-11, atol=1e-12)
    g4, _ = oracle.linear_estimate(X, c1, L, N, 0.4, 0.5, 4)
    np.testing.assert_allclose(g4 * 4.0, g1, rtol=1e-12, atol=1e-14)


def test_outer_sum_matches_matmul():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((37, 20))
    X = rng.standard_normal((37, 9))
    np.testing.assert_allclose(oracle.outer_sum(g, X), g.T @ X, rtol=1e-12, atol=1e-12)
    G1 = oracle.outer_sum(g[:1], X[:1])
    np.testing.assert_allclose(G1, np.outer(g[0], X[0]), rtol=1e-14)
    assert np.linalg.matrix_rank(G1) == 1


def test_linear_rows_agree_with_full_estimate():
    K, T, L, N, d = 6, 20, 5, 16, 4
    rng = np.random.default_rng(4)
    X = rng.standard_normal((T, d))
    c = rng.standard_normal((K, T))
    g, G = oracle.linear_estimate(X, c, L, N, 0.2, 0.9, 5)
    tok = [0, 4, 5, 19]
    np.testing.assert_allclose(oracle.linear_rows(c, L, N, 0.2, 0.9, 5, tok), g[tok],
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(G, oracle.outer_sum(g, X), rtol=1e-12)


def test_perturbed_linear_is_product_plus_noise():
    # Y[k] = X W^T + sigma a^(draw0+k): against numpy's matmul and the (pinned)
    # noise stream; linear in sigma.
    rng = np.random.default_rng(5)
    X = rng.standard_normal((9, 16))
    W = rng.standard_normal((12, 16))
    Y = oracle.perturbed_linear(X, W, 0.3, seed=4, stream=2, draw0=5, ndraw=3)
    a = oracle.noise(4, 2, 5, 3, 9, 12)
    np.testing.assert_allclose(Y, (X @ W.T)[None] + 0.3 * a, rtol=1e-12, atol=1e-12)
    Y2 = oracle.perturbed_linear(X, W, 0.6, seed=4, stream=2, draw0=5, ndraw=3)
    np.testing.assert_allclose(Y2 - Y, 0.3 * a, rtol=1e-12, atol=1e-12)


def test_term_magnitudes():
    # The oracle's per-element error scale (1/(K sigma)) sum_i (|r_i| + max_j
    # |r_j|) |a_i| (the bound that GPU rounding errors are measured against):
    # numpy from the pinned noise stream and the pinned scan, the triangle
    # inequality |g| <= scale, the closed form for a one-hot c (|g| plus the
    # one reward's size times the noise magnitudes), and the same values from
    # the rows form.
    K, T, L, N, d, sigma, gamma, seed = 6, 12, 4, 8, 3, 0.3, 0.7, 9
    rng = np.random.default_rng(6)
    X = rng.standard_normal((T, d))
    c = rng.standard_normal((K, T))
    g, _, r, s = oracle.linear_estimate(X, c, L, N, sigma, gamma, seed, with_r=True,
                                        with_scale=True)
    a = oracle.noise(seed, 0, 0, K, T, N)
    ra = np.abs(r)
    ref = ((ra + ra.max(0, keepdims=True))[:, :, None] * np.abs(a)).sum(0) / (K * sigma)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=0)
    assert (np.abs(g) <= s * (1 + 1e-12)).all()
    rows, srows = oracle.linear_rows(c, L, N, sigma, gamma, seed, [1, 7], with_scale=True)
    np.testing.assert_allclose(srows, s[[1, 7]], rtol=1e-12)
    c1 = np.zeros((K, T))
    c1[2, 5] = 1.5
    g1, _, r1, s1 = oracle.linear_estimate(X, c1, L, N, sigma, gamma, seed, with_r=True,
                                           with_scale=True)
    rmax = np.abs(r1).max(0)[:, None]
    np.testing.assert_allclose(s1, np.abs(g1) + rmax * np.abs(a).sum(0) / (K * sigma),
                               rtol=1e-12, atol=0)
