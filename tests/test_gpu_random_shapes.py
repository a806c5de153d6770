"""Seeded random shapes against the oracle: LM-head and hidden-layer estimates
whose sequence length, token count, width, vocabulary, population, discount,
sigma, dtypes, seed and stream are drawn from one generator per case (seeded
by the case number), each held to the same bar as the fixed-shape tests: whole
arrays and every row of g_hat within relative L2 1e-3 and cosine 0.99999,
every element of g_hat within its term scale, and G_W against the fp64 product
(paper digest, section 2.2, for both estimates)."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import (G_HAT_TERM_TOL, assert_elementwise, assert_gw, assert_parity, assert_rows,
                  need_gpu)

pytestmark = pytest.mark.gpu


def _shape(rng):
    L = int(rng.choice([1, 3, 16, 37, 64, 100]))
    T = L * int(rng.integers(1, 5))
    return dict(L=L, T=T, d=int(rng.integers(1, 80)), K=int(rng.integers(2, 70)),
                gamma=float(rng.choice([0.0, 0.0, 0.5, 1.0])),
                sigma=float(rng.choice([0.01, 0.05, 0.3])), bf16=bool(rng.integers(0, 2)),
                seed=int(rng.integers(0, 2**63)), stream=int(rng.integers(0, 2**32)))


@pytest.mark.parametrize("case", range(32))
def test_head_random_shape(case):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(1000 + case)
    s = _shape(rng)
    V = 4 * int(rng.integers(1, 1200))
    print(f"[random head] case {case}: {s} V={V}", flush=True)
    z, y, X = synth.head_inputs(s["T"], V, s["d"], seed=case, bf16=s["bf16"])
    g, G = dust.head_estimate(z.cuda(), y.cuda(), X.cuda(), sigma=s["sigma"], K=s["K"],
                              gamma=s["gamma"], seed=s["seed"], seq_len=s["L"],
                              stream=s["stream"])
    torch.cuda.synchronize()
    g, G = g.cpu().numpy(), G.cpu().numpy()
    rg, rG, diag = oracle.head_estimate(synth.to_f64(z), y.numpy(), synth.to_f64(X), s["L"],
                                        s["sigma"], s["K"], s["gamma"], s["seed"], s["stream"],
                                        diagnostics=True)
    assert_parity(g, rg, "g_hat")
    assert_rows(g, rg, "g_hat rows")
    assert_elementwise(g, rg, diag["g_scale"], "g_hat elements", G_HAT_TERM_TOL)
    assert_parity(G, rG, "G_W")
    assert_gw(G, rg, synth.to_f64(X))


@pytest.mark.parametrize("case", range(16))
def test_linear_random_shape(case):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(2000 + case)
    s = _shape(rng)
    N = 4 * int(rng.integers(1, 700))
    print(f"[random linear] case {case}: {s} N={N}", flush=True)
    X, c = synth.linear_inputs(s["T"], s["d"], s["K"], seed=case, c_seed=case + 1,
                               bf16=s["bf16"])
    g, G = dust.linear_estimate(X.cuda(), c.cuda(), N=N, sigma=s["sigma"], gamma=s["gamma"],
                                seed=s["seed"], seq_len=s["L"], stream=s["stream"])
    torch.cuda.synchronize()
    g, G = g.cpu().numpy(), G.cpu().numpy()
    rg, rG, sc = oracle.linear_estimate(synth.to_f64(X), c.double().numpy(), s["L"], N,
                                        s["sigma"], s["gamma"], s["seed"], s["stream"],
                                        with_scale=True)
    assert_parity(g, rg, "g_hat")
    assert_rows(g, rg, "g_hat rows")
    assert_elementwise(g, rg, sc, "g_hat elements", G_HAT_TERM_TOL)
    assert_parity(G, rG, "G_W")
    assert_gw(G, rg, synth.to_f64(X))
