"""Pins of the oracle's LM-head estimator (no GPU).

The head perturbs the cached logits and recomputes only the per-token
cross-entropy (laoyaoba analysis, mechanism section; linlog explainer, "the core
of Dust"); the credit assignment is that of the paper digest, section 2.2.
Pinned against things other than the oracle itself:
  - per-draw losses against torch's fp64 cross_entropy on the perturbed logits;
  - centring: the c of every token sums to zero over the draws and is larger
    for draws that lowered the loss;
  - the estimator's expectation: with small sigma, g_hat converges to the
    closed-form cross-entropy gradient softmax(z) - onehot(y); the token-mean
    cosine follows cos(K) = (1-1/K)/sqrt((1-1/K)^2 + (V+1)/K), which is the
    pages' fitted law cos(K) = c_max / sqrt(1 + c/K) (paper digest, section 4.2;
    linlog explainer, gradient-alignment section) with c = V+1, and the
    projection of g_hat on the gradient has mean (1 - 1/K) (sign and 1/(K sigma)
    scale);
  - the gamma = 0 identity sum_i c_i a_i = sum_i delta_i a_i - mean(delta) sum_i a_i
    that the fused GPU kernel relies on;
  - brute force on a tiny case in pure Python.
"""
import math

import numpy as np
import pytest
import torch

import oracle

V_SMALL = 512


def _inputs(T, V, d, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, V))
    y = rng.integers(0, V, T).astype(np.int32)
    X = rng.standard_normal((T, d)) / np.sqrt(d)
    return z, y, X


def _ce_grad(z, y):
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    p[np.arange(len(y)), y] -= 1.0
    return p


def test_losses_match_torch_cross_entropy():
    T, V, K, sigma, seed, stream = 24, 64, 5, 0.3, 4, 2
    z, y, X = _inputs(T, V, 8, 1)
    g, G, diag = oracle.head_estimate(z, y, X, T, sigma, K, 0.0, seed, stream, diagnostics=True)
    a = oracle.noise(seed, stream, 0, K, T, V)
    yt = torch.from_numpy(y.astype(np.int64))
    ref0 = torch.nn.functional.cross_entropy(torch.from_numpy(z), yt, reduction="none").numpy()
    np.testing.assert_allclose(diag["ell0"], ref0, rtol=0, atol=1e-12)
    for i in range(K):
        zp = torch.from_numpy(z + sigma * a[i])
        ref = torch.nn.functional.cross_entropy(zp, yt, reduction="none").numpy()
        np.testing.assert_allclose(diag["ell"][i], ref, rtol=0, atol=1e-12)


def test_centring_properties():
    T, V, K = 16, 32, 9
    z, y, X = _inputs(T, V, 4, 2)
    _, _, diag = oracle.head_estimate(z, y, X, T, 0.5, K, 0.0, 1, diagnostics=True)
    c, ell = diag["c"], diag["ell"]
    np.testing.assert_allclose(c.sum(0), 0.0, atol=1e-12)
    # a draw that lowered the loss more scores higher: c is a decrease
    for t in range(T):
        order = np.argsort(ell[:, t])
        assert np.all(np.diff(c[order, t]) <= 1e-12)
    # gamma = 0: the reward is the token's own c
    assert np.array_equal(diag["r"], c)


def test_k1_gives_zero_estimate():
    z, y, X = _inputs(8, 16, 4, 3)
    g, G = oracle.head_estimate(z, y, X, 8, 0.1, 1, 0.0, 1)
    assert np.all(g == 0) and np.all(G == 0)


def test_fused_identity():
    T, V, K, sigma = 10, 32, 7, 0.2
    z, y, X = _inputs(T, V, 4, 5)
    g, _, diag = oracle.head_estimate(z, y, X, T, sigma, K, 0.0, 8, diagnostics=True)
    a = oracle.noise(8, 0, 0, K, T, V)
    delta = diag["ell"] - diag["ell0"][None, :]
    lhs = np.einsum("it,itv->tv", diag["c"], a)
    rhs = np.einsum("it,itv->tv", delta, a) - delta.mean(0)[:, None] * a.sum(0)
    np.testing.assert_allclose(lhs, -rhs, atol=1e-12)
    np.testing.assert_allclose(g, -lhs / (K * sigma), atol=1e-12)


def test_brute_force_tiny():
    # T=2, V=4, K=3: every step in plain Python floats.
    T, V, K, sigma, gamma, L = 2, 4, 3, 0.4, 0.5, 2
    z, y, X = _inputs(T, V, 3, 6)
    a = oracle.noise(1, 0, 0, K, T, V)

    def ce(row, tgt):
        m = max(row)
        return math.log(sum(math.exp(v - m) for v in row)) + m - row[tgt]

    ell0 = [ce(list(z[t]), int(y[t])) for t in range(T)]
    ell = [[ce([z[t][v] + sigma * a[i][t][v] for v in range(V)], int(y[t])) for t in range(T)]
           for i in range(K)]
    dec = [[ell0[t] - ell[i][t] for t in range(T)] for i in range(K)]
    c = [[dec[i][t] - sum(dec[j][t] for j in range(K)) / K for t in range(T)] for i in range(K)]
    r = [[c[i][0] + gamma * c[i][1], c[i][1]] for i in range(K)]
    gh = [[-sum(r[i][t] * a[i][t][v] for i in range(K)) / (K * sigma) for v in range(V)]
          for t in range(T)]
    GW = [[sum(gh[t][v] * X[t][k] for t in range(T)) for k in range(3)] for v in range(V)]
    g, G = oracle.head_estimate(z, y, X, L, sigma, K, gamma, 1)
    np.testing.assert_allclose(g, np.array(gh), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(G, np.array(GW), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gamma", [0.0, 0.7])
def test_rows_agree_with_full_estimate(gamma):
    T, V, L, K = 12, 16, 6, 5
    z, y, X = _inputs(T, V, 4, 7)
    g, _ = oracle.head_estimate(z, y, X, L, 0.3, K, gamma, 2)
    tok = [0, 3, 5, 6, 11]
    rows = oracle.head_rows(z, y, L, 0.3, K, gamma, 2, tok)
    np.testing.assert_allclose(rows, g[tok], rtol=1e-12, atol=1e-14)
    # the error scales (1/(K sigma)) sum_i (|r_i| + max_j |r_j|) |a_i|: the rows
    # form agrees with the full estimate's, and numpy rebuilds them from r and
    # the noise
    _, _, diag = oracle.head_estimate(z, y, X, L, 0.3, K, gamma, 2, diagnostics=True)
    rows2, srows = oracle.head_rows(z, y, L, 0.3, K, gamma, 2, tok, with_scale=True)
    np.testing.assert_allclose(srows, diag["g_scale"][tok], rtol=1e-12, atol=1e-14)
    a = oracle.noise(2, 0, 0, K, T, V)
    r = np.abs(diag["r"])
    ref = ((r + r.max(0, keepdims=True))[:, :, None] * np.abs(a)).sum(0) / (K * 0.3)
    np.testing.assert_allclose(diag["g_scale"], ref, rtol=1e-12, atol=1e-14)
    assert (np.abs(g) <= diag["g_scale"] * (1 + 1e-12)).all()


def _cos_rows(a, b):
    return np.sum(a * b, 1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def _predicted_cos(K, V):
    k = 1 - 1 / K
    return k / np.sqrt(k * k + (V + 1) / K)


@pytest.mark.parametrize("sigma", [0.05, 0.005])
def test_estimate_converges_to_ce_gradient(sigma):
    # The pages' convergence claim (paper digest, section 4.2): the estimate's
    # cosine with the backprop gradient rises with the population.  For the
    # head the backprop gradient is softmax(z) - onehot(y).
    T, V = 32, V_SMALL
    z, y, X = _inputs(T, V, 8, 11)
    gref = _ce_grad(z, y)
    means = {}
    for K, seed in ((16, 21), (256, 22), (4096, 23)):
        g, _ = oracle.head_estimate(z, y, X, T, sigma, K, 0.0, seed)
        cos = _cos_rows(g, gref)
        se = cos.std(ddof=1) / np.sqrt(T)
        means[K] = cos.mean()
        assert abs(cos.mean() - _predicted_cos(K, V)) < 3 * se + 0.01, (K, cos.mean(), se)
        beta = np.sum(g * gref, 1) / np.sum(gref * gref, 1)
        bse = np.sqrt(2.0 / K) / np.sqrt(T)
        assert abs(beta.mean() - (1 - 1 / K)) < 4 * bse + 0.01, (K, beta.mean(), bse)
    assert means[16] < means[256] < means[4096]


def test_cosine_law_fit():
    # Fit cos(K) = c_max / sqrt(1 + c/K) on oracle estimates (sigma small):
    # c lands within 20% of V+1 and c_max near 1.
    from scipy.optimize import curve_fit
    T, V, sigma = 16, V_SMALL, 0.005
    z, y, X = _inputs(T, V, 8, 12)
    gref = _ce_grad(z, y)
    Ks = np.array([16, 64, 256, 1024, 4096, 16384])
    cs = []
    for n, K in enumerate(Ks):
        g, _ = oracle.head_estimate(z, y, X, T, sigma, int(K), 0.0, 100 + n)
        cs.append(_cos_rows(g, gref).mean())
    (cmax, c), _ = curve_fit(lambda k, cm, cc: cm / np.sqrt(1 + cc / k), Ks.astype(float),
                             np.array(cs), p0=(1.0, 500.0))
    assert 0.8 * (V + 1) <= c <= 1.2 * (V + 1), (cmax, c, cs)
    assert cmax >= 0.99, (cmax, c, cs)
    # G_W's cosine with the closed-form weight gradient grows the same way
    Gref = gref.T @ X
    gk, Gk = oracle.head_estimate(z, y, X, T, sigma, 4096, 0.0, 7)
    g16, G16 = oracle.head_estimate(z, y, X, T, sigma, 16, 0.0, 8)
    cw = lambda A, B: float(np.sum(A * B) / np.linalg.norm(A) / np.linalg.norm(B))
    assert cw(Gk, Gref) > cw(G16, Gref) and cw(Gk, Gref) > 0.9


def test_one_token_sequences_make_the_discount_irrelevant():
    # With seq_len = 1 every token is its own sequence: r_t = c_t whatever gamma,
    # so the estimate equals the gamma = 0 one (paper digest, section 2.2: the
    # discounted sum runs over later tokens of the same sequence only).
    z, y, X = _inputs(24, 64, 8, seed=21)
    g0, G0 = oracle.head_estimate(z, y, X, 24, 0.05, 6, 0.0, 3)
    g1, G1 = oracle.head_estimate(z, y, X, 1, 0.05, 6, 0.9, 3)
    assert np.allclose(g1, g0, rtol=1e-12, atol=1e-15)
    assert np.allclose(G1, G0, rtol=1e-12, atol=1e-15)
