"""dust_linear_estimate (hidden linear layer, caller-supplied centred loss
decreases) against the oracle, and the closed form for a one-hot c:
g_t = -(1/(K sigma)) gamma^(s-t) a_t for t <= s in s's sequence, 0 elsewhere
(paper digest, section 2.2), with a from the oracle's noise stream."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import (G_HAT_TERM_TOL, assert_elementwise, assert_gw, assert_parity, assert_rows,
                  need_gpu)

pytestmark = pytest.mark.gpu


def _run(dust, X, c, **kw):
    import torch
    g, G = dust.linear_estimate(X.cuda(), c.cuda(), **kw)
    torch.cuda.synchronize()
    return g.cpu().numpy(), G.cpu().numpy()


@pytest.mark.parametrize("T,L,d,N,K,gamma,bf16", [
    (256, 64, 96, 200, 10, 0.9, False), (256, 64, 96, 200, 10, 0.9, True),
    (300, 300, 40, 2048, 7, 0.0, True), (120, 40, 17, 12, 66, 1.0, False),
    (64, 8, 64, 8192, 3, 0.5, True)])
def test_linear_matches_oracle(T, L, d, N, K, gamma, bf16):
    dust = need_gpu()
    X, c = synth.linear_inputs(T, d, K, seed=T + N, c_seed=K, bf16=bf16)
    sigma, seed, stream = 0.01, 9, 1
    g, G = _run(dust, X, c, N=N, sigma=sigma, gamma=gamma, seed=seed, seq_len=L, stream=stream)
    rg, rG, sc = oracle.linear_estimate(synth.to_f64(X), c.double().numpy(), L, N, sigma, gamma,
                                        seed, stream, with_scale=True)
    assert_parity(g, rg, "g_hat")
    assert_rows(g, rg, "g_hat rows")
    assert_elementwise(g, rg, sc, "g_hat elements", G_HAT_TERM_TOL)
    assert_parity(G, rG, "G_W")
    assert_gw(G, rg, synth.to_f64(X))


def test_one_hot_closed_form():
    dust = need_gpu()
    import torch
    T, L, N, K, d, sigma, gamma, seed = 64, 16, 40, 5, 8, 0.05, 0.8, 123
    a = oracle.noise(seed, 0, 0, K, T, N)
    X = torch.ones((T, d), dtype=torch.float32)
    for (i_s, s_s) in ((3, 37), (0, 16), (4, 63)):
        c = torch.zeros((K, T), dtype=torch.float32)
        c[i_s, s_s] = 1.0
        g, _ = _run(dust, X, c, N=N, sigma=sigma, gamma=gamma, seed=seed, seq_len=L)
        ref = np.zeros((T, N))
        for t in range((s_s // L) * L, s_s + 1):
            ref[t] = -(gamma ** (s_s - t)) * a[i_s, t] / (K * sigma)
        assert_parity(g, ref, "g_hat one-hot")
        inside = ~np.all(ref == 0, axis=1)
        assert_rows(g[inside], ref[inside], "g_hat one-hot rows")
        # one term per element: within fp32 rounding of the scan's powers of
        # gamma, plus the normals' own accuracy (1e-5 absolute) times 1/(K sigma)
        assert_elementwise(g, ref, np.abs(ref), "g_hat one-hot elements", 1e-5,
                           atol=1e-5 / (K * sigma))
        outside = np.ones(T, bool)
        outside[(s_s // L) * L:s_s + 1] = False
        assert np.all(g[outside] == 0)
